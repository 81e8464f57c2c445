// common.hpp -- device-side building blocks shared by the SpliceGEMM kernels
// (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace splice {

typedef _Float16 f16;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int WAVE = 64;
constexpr int NVFP4_BLOCK = 16;

// ---------------------------------------------------------------------------
// Exact NVFP4 -> FP16 decode.
//
// An E2M1 value (at most 2 significant bits) times an E4M3 block scale (4
// significant bits, 2^-9 .. 448) has at most 6 significant bits and lies in
// [2^-10, 2688]: it is exactly representable as an FP16 normal number.  The
// gfx950 FP4 conversion applies only the exponent of its scale operand, so the
// codes are converted with scale 1.0 and the E4M3 scale is applied with a
// packed FP16 multiply, which is exact because the product is representable.
// ---------------------------------------------------------------------------

// (s, s) as FP16 from one E4M3FN byte.
__device__ __forceinline__ f16x2 e4m3_pair(unsigned byte)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte * 0x0101u, 1.0f, false);
}

// 8 FP4 codes (one dword, code 0 in bits 3:0) times scale pair -> 8 FP16 values
// in channel order, as one MFMA operand.
__device__ __forceinline__ f16x8 decode8(unsigned codes, f16x2 sc)
{
    f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sc;
    f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sc;
    f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sc;
    f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sc;
    return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// v_mfma_f32_16x16x32_{f16,bf16}: lane l holds row (l%16) of A and column
// (l%16) of B at reduction indices 8*(l/16) .. +8; the 16x16 result in lane l
// is rows 4*(l/16) .. +4 of column l%16.
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(16))) float f32x16;

// v_mfma_f32_32x32x16_{f16,bf16}: lane l holds row (l%32) of A and column
// (l%32) of B at reduction indices 8*(l/32) .. +8; result element q of lane l
// is row 8*(q/4) + 4*(l/32) + q%4 of column l%32.
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier that makes this wave's LDS writes visible but, unlike
// __syncthreads(), does not wait for outstanding global loads (the fence of
// __syncthreads() would drain a prefetch issued for a later pipeline stage).
// The wait and the barrier builtins touch no memory as far as the compiler's
// IR passes know, so an empty asm statement with a memory clobber on each side
// keeps LDS loads and stores from being moved across the barrier; the
// scheduling barrier does the same for the machine scheduler.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left at their maximum
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(0): every global load and store this wave has issued has
// completed (for a device-coherent store: it is visible to every workgroup).
__device__ __forceinline__ void wait_vmem()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt left at their maximum
    asm volatile("" ::: "memory");
}

// Device-coherent 16-byte accesses for partial sums exchanged between
// workgroups: raw buffer loads and stores with the sc1 cache policy, the
// policy the compiler gives agent-scope relaxed atomics (they bypass the
// per-XCD caches that are not coherent with each other), but twice as wide
// as a 64-bit atomic and free to be scheduled like ordinary loads.  The
// resource covers `bytes` bytes from `base`; offsets past it read 0 and
// write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ u32x4 coherent_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CPOL_SC1));
}
__device__ __forceinline__ void coherent_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, CPOL_SC1);
}

// 8 bf16 values (16 bytes) of a side buffer row, zero past `valid` elements.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p, int valid, bool aligned16)
{
    if (valid >= 8 && aligned16) {
        u32x4 v = *reinterpret_cast<const u32x4 *>(p);
        return __builtin_bit_cast(bf16x8, v);
    }
    uint16_t t[8];
#pragma unroll
    for (int i = 0; i < 8; i++) t[i] = (i < valid) ? p[i] : (uint16_t)0;
    u32x4 v;
    v.x = t[0] | ((unsigned)t[1] << 16);
    v.y = t[2] | ((unsigned)t[3] << 16);
    v.z = t[4] | ((unsigned)t[5] << 16);
    v.w = t[6] | ((unsigned)t[7] << 16);
    return __builtin_bit_cast(bf16x8, v);
}

}  // namespace splice
