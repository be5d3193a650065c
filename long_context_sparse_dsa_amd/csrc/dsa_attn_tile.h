// dsa_attn_tile.h -- device pieces shared by the attention kernels: the
// exp2 / reciprocal / sigmoid helpers, the LDS transpose read and the
// swizzled K / V row tile (used by dsa_attn.hip and by the fused decode
// selection + attention kernel in dsa_topk.hip).
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp), which
// keep the latency-bound epilogues short; the outputs are bf16.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoidf(float x) { return frcp(1.f + fexp2(-x * kLog2e)); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 8 bytes addressed by lane 4e + i/4, for e = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  u32x2 r;
  r[0] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
  r[1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
  return r;
}

// A 32-row tile of K or V rows in LDS: row-major (2D bytes per row), its
// 16-byte chunks permuted within each row by an XOR with f(r), a bijection
// of r mod NC (NC = D / 8 chunks per row).  The accesses made of it stay
// free of bank conflicts:
//   - gathers write whole rows (one row's NC chunks per NC lanes): XOR with
//     a constant permutes the chunks of a row;
//   - the K operand reads one chunk of 8 or 16 consecutive rows per LDS
//     pass: f takes distinct values there, so the chunks land on distinct
//     16-byte slots (32 or 64 banks);
//   - the V transpose reads 8 bytes of two neighbouring chunks (c even,
//     c + 1) of 4 aligned consecutive rows per 16 lanes: bits 1-2 of f
//     differ over such rows, so the 8 slots differ.
// Gathers: with RPI = 64 / NC rows per load instruction, instruction c of
// a tile reads rows RPI c + l / NC, chunk l % NC: each instruction covers
// RPI whole rows (RPI x 2D bytes), the fewest cache lines a 1 KiB load can
// touch, where a lane-per-row layout would touch 32 rows.
template <int D>
struct RowTile {
  static constexpr int kNC = D / 8;            // 16-byte chunks per row
  static constexpr int kRPI = 64 / kNC;        // rows per load instruction
  static constexpr int kLoads = 32 / kRPI;     // load instructions per tile
  static constexpr int kBytes = 32 * D * 2;
  // bits 1-2 of f(r) are r mod 4, bit 0 is bit 2 of r, bit 3 (kNC = 16) is
  // bit 3 of r: a bijection whose low three bits differ over any 8 aligned
  // rows (K operand reads, 8 or 16 lanes per LDS pass) and whose bits 1-2
  // differ over any 4 aligned rows (V transposes)
  __device__ static int swz(int r) {
    return (((r & 3) << 1) | ((r >> 2) & 1) | (r & 8)) & (kNC - 1);
  }
  // byte offset of element (row r, dim d)
  __device__ static int offset(int r, int d) {
    return r * (2 * D) + ((((d >> 3) ^ swz(r)) << 4) | ((d & 7) << 1));
  }
};

}  // namespace dsa
