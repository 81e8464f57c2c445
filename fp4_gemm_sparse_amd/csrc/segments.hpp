// segments.hpp -- launches over column segments: the products of one set of
// activation operands with several weight matrices (splice_gemm_multi and
// its fused-preparation form), one kernel launch.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace splice {

// ===========================================================================
// Column segments: products that share the activation operands (X, its
// packs and X_S) but each have their own weights, tensor scale and output --
// the q, k and v projections of one layer input, say -- computed by one
// launch.  The launch units of a kernel (tile columns, column blocks) are
// numbered across the segments in order and never straddle two, so each unit
// runs exactly the code of a call on its own segment.
// ===========================================================================
struct SegTable {
    GemmArgs a;                          // shared operands, M, K, k
    GemmSeg seg[SEG_MAX];
    int start[SEG_MAX + 1];              // first unit of each segment; start[nseg] = all units
    int nseg;
};

inline SegTable make_seg_table(const GemmArgs &a, const SegSpec &sp, int64_t unit)
{
    SegTable t;
    t.a = a;
    t.nseg = sp.nseg;
    t.start[0] = 0;
    for (int i = 0; i < SEG_MAX; i++) {
        t.seg[i] = i < sp.nseg ? sp.seg[i] : sp.seg[0];
        if (i < sp.nseg) t.start[i + 1] = t.start[i] + (int)((sp.seg[i].N + unit - 1) / unit);
    }
    for (int i = sp.nseg + 1; i <= SEG_MAX; i++) t.start[i] = t.start[sp.nseg];
    return t;
}

// the arguments of unit u's segment, and u's index inside it
__device__ __forceinline__ GemmArgs seg_args(const SegTable &t, int u, int &local)
{
    int sg = 0;
#pragma unroll
    for (int i = 1; i < SEG_MAX; i++)
        if (i < t.nseg && u >= t.start[i]) sg = i;
    local = u - t.start[sg];
    GemmArgs r = t.a;
    const GemmSeg &w = t.seg[sg];
    r.Wq = w.Wq;
    r.Ws = w.Ws;
    r.alpha_w = w.alpha_w;
    r.W_S = w.W_S;
    r.Y = w.Y;
    r.ldy = w.ldy;
    r.N = w.N;
    return r;
}

}  // namespace splice
