// dsa_device.h -- gfx950 device helpers shared by the DSA kernels.
//
// MFMA operand layouts used throughout (wave64, checked on gfx950):
//   v_mfma_f32_32x32x16_bf16  A[i][k]: lane l holds row i = l%32, k = 8*(l/32)+0..7
//                             B[k][j]: lane l holds col j = l%32, k = 8*(l/32)+0..7
//                             C[i][j]: lane l, reg r holds i = 8*(r/4)+4*(l/32)+r%4, j = l%32
// Because every contraction below sums over k, the kernels are free to assign
// any fixed permutation of the contracted dimension to the k slots, as long
// as both operands use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef int v8i32 __attribute__((ext_vector_type(8)));

// fp8 MFMA (E4M3FN x E4M3FN, 32x32x64, fp32 accumulation).  Operands: 32
// bytes per lane, row / column l % 32, k slots 32 (l / 32) + 0..31; C as in
// mfma32.  Zero scale operands select the unscaled instruction.
__device__ __forceinline__ f32x16 mfma_f8(const v8i32& a, const v8i32& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Order-preserving map of an fp32 score onto uint32: larger key <=> larger
// value, with -0.0 mapped onto +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t x = __float_as_uint(f);
  if (x == 0x80000000u) x = 0u;
  return (x & 0x80000000u) ? ~x : (x | 0x80000000u);
}

// 16 bytes holding 8 bf16 -> MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// 8 fp8 e4m3fn codes (two dwords) -> 8 bf16, exact (every e4m3fn value is a
// bf16 value; the gfx950 conversion with scale 1.0 is exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Direct global->LDS loads (global_load_lds_dword{,x4}): lane l's bytes land
// at lds + size * l, where `lds` must be the same for the whole wave.  The
// load counts in vmcnt until its data is in LDS.  (Kept in plain functions:
// the builtin used directly inside a kernel template stops the host pass
// from emitting that kernel's launch stub.)
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
}
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---------------------------------------------------------------------------
// Cross-lane primitives.  A dependent ds_bpermute (__shfl_*) costs about 136
// cycles on gfx950 and a ballot + popcount step about 72; DPP row moves and
// v_permlane32_swap are VALU operations of a few cycles, so the wave-wide
// scans and reductions below are built from them.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, ROW_MASK, BANK_MASK,
                                               false);
}

// The value of lane l^32 (the other half of the wave).
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (lane_id() < 32) ? (uint32_t)r[1] : (uint32_t)r[0];
}
// Sum / max across the two 32-lane halves of a wave (same result in both).
__device__ __forceinline__ float xor32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float((uint32_t)r[0]) + __uint_as_float((uint32_t)r[1]);
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float((uint32_t)r[0]), __uint_as_float((uint32_t)r[1]));
}

// Inclusive wave scan with an associative operator op and identity id:
// row shifts 1, 2, 4, 8 build 16-lane row scans, two row broadcasts join
// the rows.
// Every lane of a quad (4 aligned lanes) gets lane K of the quad.
template <int K>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, K * 0x55, 0xf, 0xf, false);
}

template <typename Op>
__device__ __forceinline__ uint32_t dpp_wave_scan(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp_u32<kDppRowShr1, 0xf, 0xf>(id, v));
  v = op(v, dpp_u32<kDppRowShr2, 0xf, 0xf>(id, v));
  v = op(v, dpp_u32<kDppRowShr4, 0xf, 0xf>(id, v));
  v = op(v, dpp_u32<kDppRowShr8, 0xf, 0xf>(id, v));
  v = op(v, dpp_u32<kDppRowBcast15, 0xa, 0xf>(id, v));
  v = op(v, dpp_u32<kDppRowBcast31, 0xc, 0xf>(id, v));
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  return dpp_wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  const uint32_t s = dpp_wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)s, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  const uint32_t s =
      dpp_wave_scan(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)s, 63);
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  const uint32_t s = dpp_wave_scan(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)s, 63));
}
__device__ __forceinline__ int32_t wave_max_i32(int32_t v) {
  // order-preserving bias so the unsigned maximum is the signed one
  return (int32_t)(wave_max_u32((uint32_t)v ^ 0x80000000u) ^ 0x80000000u);
}
__device__ __forceinline__ float wave_max_f32(float v) {
  // monotone map of fp32 onto uint32 (no NaN in use)
  uint32_t x = __float_as_uint(v);
  x = (x & 0x80000000u) ? ~x : (x | 0x80000000u);
  x = wave_max_u32(x);
  x = (x & 0x80000000u) ? (x & 0x7fffffffu) : ~x;
  return __uint_as_float(x);
}

// max(x, 0) as one integer max on the bit pattern: every float with the
// sign bit set (negative values, -0.0) becomes +0.0, the rest pass.  fmaxf
// would first canonicalize x (a second instruction per element).
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every outstanding global load and store of the wave (vmcnt(0));
// none of the barriers in these kernels protects global memory, so they use
// this one and keep global traffic in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier that waits only for this wave's own LDS instructions.
// The release fence of lds_barrier() also waits for every direct
// global-to-LDS load still in flight (they count as LDS writes) and for the
// wave's global stores, which empties a prefetch pipeline at every barrier.
// Waves that order their direct loads with explicit vmcnt waits, or only
// have stores in flight, use this one; the empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Exclusive block-wide prefix sum of one value per thread.  `scratch` holds
// at least blockDim.x/64 + 1 uint32.  Returns the exclusive prefix; *total
// receives the block total.  The cross-wave step runs in wave 0's registers
// (no serial chain through LDS).  Contains barriers: call from every thread.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int w = wave_id(), nw = blockDim.x >> 6, l = lane_id();
  const uint32_t inc = wave_incl_scan(v);
  if (l == 63) scratch[w] = inc;
  lds_barrier();
  if (w == 0) {
    const uint32_t x = l < nw ? scratch[l] : 0u;
    const uint32_t xs = wave_incl_scan(x);
    if (l < nw) scratch[l] = xs - x;
    if (l == 63) scratch[nw] = xs;
  }
  lds_barrier();
  const uint32_t r = scratch[w] + inc - v;
  *total = scratch[nw];
  lds_barrier();
  return r;
}

// ---------------------------------------------------------------------------
// fp8 indexer key cache: OCP E4M3FN codes plus one fp32 scale per token (the
// naive-n0-5-flash page, Key Capabilities: FP8).  The scale is the row's
// absolute maximum over 448, the format's largest finite value, and each
// element is rounded to the nearest code, ties to even, from its fp32
// quotient by the scale clamped to +-448.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);  // multiples of 2^-9; 8 -> 0x08
  const uint32_t au = __float_as_uint(a);
  int e = (int)(au >> 23) - 127;  // -6 .. 8
  const uint32_t mant = au & 0x7fffffu;
  uint32_t m3 = mant >> 20;
  const uint32_t rest = mant & 0xfffffu;
  m3 += (uint32_t)(rest > 0x80000u) | ((uint32_t)(rest == 0x80000u) & (m3 & 1u));
  if (m3 == 8u) {
    ++e;
    m3 = 0;
  }
  return sign | ((uint32_t)(e + 7) << 3) | m3;
}

// Quantise one indexer key row held two elements per lane (x0, x1 = row
// elements 2 l, 2 l + 1): returns the two codes packed in 16 bits (element
// 2 l in the low byte) and the row's scale.
__device__ __forceinline__ uint32_t e4m3_row_pair(float x0, float x1, float* sigma_out) {
  const uint32_t m = wave_max_u32(max(__float_as_uint(fabsf(x0)), __float_as_uint(fabsf(x1))));
  const float amax = __uint_as_float(m);
  const float sigma = amax > 0.f ? amax / 448.f : 1.f;
  const float y0 = fminf(fmaxf(x0 / sigma, -448.f), 448.f);
  const float y1 = fminf(fmaxf(x1 / sigma, -448.f), 448.f);
  *sigma_out = sigma;
  return e4m3_code(y0) | (e4m3_code(y1) << 8);
}

// Position of query row t: decode (cu_q == nullptr) has one query per
// sequence at position ctx_len-1; otherwise query i of sequence b sits at
// ctx_len[b] - n_q[b] + i.
struct RowInfo {
  int b;
  int64_t p;
};

__device__ __forceinline__ RowInfo row_info(int t, const int32_t* cu_q, const int32_t* ctx_len,
                                            int B) {
  RowInfo r;
  if (cu_q == nullptr) {
    r.b = t;
    r.p = (int64_t)ctx_len[t] - 1;
    return r;
  }
  int lo = 0, hi = B - 1;  // last b with cu_q[b] <= t
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  r.b = lo;
  r.p = (int64_t)ctx_len[lo] - (cu_q[lo + 1] - cu_q[lo]) + (t - cu_q[lo]);
  return r;
}

}  // namespace dsa
