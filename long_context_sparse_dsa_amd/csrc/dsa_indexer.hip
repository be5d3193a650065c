// dsa_indexer.hip -- Indexer scores on gfx950 MFMA.
//
// The Indexer is a lightweight multi-head scorer of every causal past
// position ("Open-Source LLM Architecture Evolution ...", Architecture
// Breakdown item 2; "Fine-Grained Sparse Attention ...", 2.2: no RoPE, 2.3:
// 32 heads x 128 dim; the naive-n0-5-flash page: 16-head indexer):
//
//   s[t, j] = sum_h w[t,h] * max(0, sigma_j * q_idx[t,h,:] . k_idx[j,:])
//
// Both kernels run the per-head dot products as bf16 MFMA contractions with
// fp32 accumulation (v_mfma_f32_32x32x16_bf16).  fp8 e4m3fn keys are widened
// to bf16 in registers (exact), so fp8 only changes the bytes streamed.
//
// Decode (one query per sequence): HBM-bound stream of the key cache.
//   A = the query's heads (32 rows, zero-padded), B = 32 keys per block.
//   Each lane loads its key row's 16-byte chunks straight into MFMA operand
//   registers (no LDS round trip); C holds one key per lane column, so the
//   ReLU / head-weight / head-sum epilogue is 16 fused multiply-adds in
//   registers plus one cross-half add.  The workgroup's tile of scores is
//   then kept in LDS for the Top-K candidate report (dsa_topk_tile.h).
//
// Prefill (a chunk of queries per sequence): MFMA-bound dense contraction.
//   A = (query, head) rows of several queries, B = key tile staged in LDS
//   and shared by the four waves; rows are assigned so that every lane's 16
//   accumulator rows are whole queries, keeping the head sum in registers.
//   Key tiles past the last visible position of the workgroup's queries are
//   skipped; the diagonal tile is masked.
#include <hip/hip_ext.h>

#include "dsa_kernels.h"
#include "dsa_topk_tile.h"

#include <cmath>
#include <mutex>
#include <type_traits>

namespace dsa {

// Offset (in elements) of the 8 consecutive dims a lane of half `g` feeds
// into k-step s.  bf16 rows: natural order.  fp8 rows: each lane reads one
// 16-byte chunk covering two k-steps.
template <bool FP8>
__device__ __forceinline__ int kslot_dim(int s, int g) {
  return FP8 ? (32 * (s >> 1) + 16 * g + 8 * (s & 1)) : (16 * s + 8 * g);
}

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------
// One wave per tile of TILE keys.  The key rows are streamed through LDS
// with global_load_lds_dwordx4: every load instruction reads 1 KiB of
// consecutive rows (fully coalesced) and lands it in LDS, where a per-KiB pad
// and a (row, chunk) lane permutation make the MFMA-operand reads free of
// bank conflicts.  The tile is cut into stages of at most 16 KiB, three of
// them in flight (a wave keeps under 64 loads outstanding, the limit of its
// load counter): while stage s is consumed, stages s+1 and s+2 are loading.  Each
// 32-key block is consumed as soon as its own loads have landed (vmcnt counts
// completions in issue order).  Scores stay in registers until the end, and
// with REPORT the wave writes the tile's Top-K candidate prefix
// (dsa_topk_tile.h) without any cross-wave step.
template <int ROWB, int TILE, bool FP8, bool DEEP>
struct KeyStage {
  static constexpr int kTileBytes = TILE * ROWB;
  // Two shapes: DEEP (few tiles per CU): stages of at most 16 KiB, three in
  // flight, so each wave keeps up to 48 KiB of loads outstanding; otherwise
  // stages of at most 8 KiB, two in flight, and more waves fit in LDS.
  // (fp8: at most 128 keys per stage, whose scales take two more loads.)
  static constexpr int kMax = DEEP ? 16384 : 8192;
  static constexpr int kCap = FP8 && 128 * ROWB < kMax ? 128 * ROWB : kMax;
  static constexpr int kBytes = kTileBytes < kCap ? kTileBytes : kCap;
  static constexpr int kNum = kTileBytes / kBytes;       // stages per tile
  static constexpr int kDepth = DEEP ? 3 : 2;
  static constexpr int kBufs = kNum < kDepth ? kNum : kDepth;  // LDS stage buffers, all in flight
  static constexpr int kRows = kBytes / ROWB;            // keys per stage
  static constexpr int kRowsPerKiB = 1024 / ROWB;        // rows per load instruction
  static constexpr int kPad = kRowsPerKiB >= 16 ? 0 : 256 / kRowsPerKiB;  // bytes per KiB
  static constexpr int kStride = 1024 + kPad;            // LDS bytes per KiB of keys
  static constexpr int kKeyBytes = (kBytes / 1024) * kStride;
  static constexpr int kScaleLoads = FP8 ? kRows / 64 : 0;  // 4-byte scale loads per stage
  static constexpr int kBufBytes = kKeyBytes + (FP8 ? 4 * kRows : 0);
  static constexpr int kKeyLoads = kBytes / 1024;        // key load instructions per stage
  static constexpr int kLoads = kKeyLoads + kScaleLoads; // load instructions per stage
  // LDS byte offset of 16-byte chunk `ck` of stage row r
  __device__ static int offset(int r, int ck) {
    return (r / kRowsPerKiB) * kStride + (ck * kRowsPerKiB + r % kRowsPerKiB) * 16;
  }
};

// s_waitcnt vmcnt(n) for an n that is a constant after unrolling (the
// builtin needs an immediate; the switch folds away).
// gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14].
#define DSA_WAITV(N) \
  case N: __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14)); break;
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    DSA_WAITV(0) DSA_WAITV(1) DSA_WAITV(2) DSA_WAITV(3) DSA_WAITV(4) DSA_WAITV(5) DSA_WAITV(6)
    DSA_WAITV(7) DSA_WAITV(8) DSA_WAITV(9) DSA_WAITV(10) DSA_WAITV(11) DSA_WAITV(12)
    DSA_WAITV(13) DSA_WAITV(14) DSA_WAITV(15) DSA_WAITV(16) DSA_WAITV(17) DSA_WAITV(18)
    DSA_WAITV(19) DSA_WAITV(20) DSA_WAITV(21) DSA_WAITV(22) DSA_WAITV(23) DSA_WAITV(24)
    DSA_WAITV(25) DSA_WAITV(26) DSA_WAITV(27) DSA_WAITV(28) DSA_WAITV(29) DSA_WAITV(30)
    DSA_WAITV(31) DSA_WAITV(32) DSA_WAITV(33) DSA_WAITV(34) DSA_WAITV(35) DSA_WAITV(36)
    DSA_WAITV(37) DSA_WAITV(38) DSA_WAITV(39) DSA_WAITV(40) DSA_WAITV(41) DSA_WAITV(42)
    DSA_WAITV(43) DSA_WAITV(44) DSA_WAITV(45) DSA_WAITV(46) DSA_WAITV(47) DSA_WAITV(48)
    DSA_WAITV(49) DSA_WAITV(50) DSA_WAITV(51) DSA_WAITV(52) DSA_WAITV(53) DSA_WAITV(54)
    DSA_WAITV(55) DSA_WAITV(56) DSA_WAITV(57) DSA_WAITV(58) DSA_WAITV(59) DSA_WAITV(60)
    DSA_WAITV(61) DSA_WAITV(62) DSA_WAITV(63)
    default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;
  }
}
#undef DSA_WAITV

// With APPEND the kernel also performs the cache append of each sequence's
// new token (position p = ctx_len - 1): the wave whose key range holds p
// loads the new rows before anything else, patches row p of its LDS stage
// (the new key, quantised for an fp8 cache) before scoring it, and writes
// the rows into the caches after its last load was consumed (a store in
// flight would disturb the exact load counts of the waits).  Only this wave
// uses row p's score; the attention reads K / V in a later kernel.  The key
// cache is then written by this kernel, so k_idx / k_scale are not
// declared restrict.
template <int DI, bool FP8, int TILE, bool REPORT, bool DEEP, int WPT, bool APPEND>
__global__ __launch_bounds__(64 * WPT) void index_decode_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w, int64_t w_ld,
    const uint8_t* k_idx, const float* k_scale, int H_I,
    const int32_t* __restrict__ ctx_len, const int64_t* __restrict__ cu_ctx,
    float* __restrict__ scores, int64_t ld, RepHeader* hdr, uint32_t* rep_u, int32_t* rep_j,
    int stride, int topk, DecodeAppend app) {
  constexpr int KS = DI / 16;                       // MFMA k-steps
  constexpr int ROWB = FP8 ? DI : 2 * DI;           // bytes per key row
  constexpr int TW = TILE / WPT;                    // keys per wave
  using St = KeyStage<ROWB, TW, FP8, DEEP>;
  constexpr int NSTAGE = St::kNum;
  constexpr int SROWS = St::kRows;
  constexpr int SBLK = SROWS / 32;                  // 32-key blocks per stage
  constexpr int NI = St::kKeyLoads;                 // key load instructions per stage
  constexpr int NL = St::kLoads;                    // all load instructions per stage
  constexpr int IPB = NI / SBLK;                    // key load instructions per block
  constexpr int NLD = FP8 ? KS / 2 : KS;            // 16-byte operand chunks per lane per block
  constexpr int V = TILE / 64;                      // report values per lane
  constexpr int VW = TW / 64;                       // stored values per lane and wave
  static_assert(KS + 1 + St::kBufs * NL <= 63 && NI % SBLK == 0 && TW % SROWS == 0,
                "stage shape");
  static_assert(KS % WPT == 0, "query rows split over the waves");

  // One LDS object (with several objects the compiler adds a wait for every
  // load in flight before reading any of them):
  //   [query rows | head weights] [tile scores] [stage buffers of wave 0 | 1 ..]
  // A single wave has its query rows and weights in registers before it
  // writes its first score (LDS operations of one wave run in order), so
  // there the scores overlay the query region: less LDS per workgroup, more
  // workgroups (loads in flight) per CU.  Several waves read the shared
  // query region at their own pace, so they keep the regions apart.
  constexpr int kQwBytes = 1024 * KS + 256;
  constexpr int kScOff = WPT == 1 ? 0 : kQwBytes;
  constexpr int kStageOff = (kScOff + 4 * TILE) > kQwBytes ? (kScOff + 4 * TILE) : kQwBytes;
  constexpr int kWaveStage = St::kBufs * St::kBufBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStageOff + WPT * kWaveStage];
  uint8_t* const qw_lds = lds;
  float* const sc_lds = reinterpret_cast<float*>(lds + kScOff);

  const int b = blockIdx.y, ti = blockIdx.x;
  // both descriptor loads issued together (one round trip)
  const int64_t row0 = cu_ctx[b];
  const int64_t p = (int64_t)ctx_len[b] - 1;
  const int64_t j0 = (int64_t)ti * TILE;
  // (testing row0 here keeps its load ahead of the branch, in the same round trip)
  if (j0 > p || row0 < 0) return;
  const int n_valid = (int)min<int64_t>(TILE, p + 1 - j0);
  const int l = lane_id(), g = l >> 5, wv = WPT > 1 ? wave_id() : 0;
  const int64_t jw0 = j0 + wv * TW;               // first key of this wave
  uint8_t* const stage = lds + kStageOff + wv * kWaveStage;

  // fused cache append: the wave holding position p loads the new rows first
  // (the oldest loads, so every later wait covers them)
  [[maybe_unused]] bool own = false;
  [[maybe_unused]] int r_p = 0;           // p's row within this wave's range
  [[maybe_unused]] uint32_t kpair = 0;    // new key elements 2 l, 2 l + 1 (bf16)
  [[maybe_unused]] u32x4 kvrow = {};      // new K (lanes < D/8) or V chunk
  if constexpr (APPEND) {
    own = p >= jw0 && p < jw0 + TW;  // wave-uniform
    if (own) {
      r_p = (int)(p - jw0);
      if (2 * l < DI) kpair = *reinterpret_cast<const uint32_t*>(app.k_idx_new + (int64_t)b * DI + 2 * l);
      const int nc = app.D / 8;
      const bool is_v = l >= nc;
      const uint16_t* src = is_v ? app.v_new : app.k_new;
      if (l < 2 * nc && src != nullptr) kvrow = ld16(src + (int64_t)b * app.D + 8 * (is_v ? l - nc : l));
    }
  }

  // A operand: query heads (rows).  Rows past H_I repeat the last head and
  // get head weight 0, so they add nothing.  The query rows and the head
  // weights go through LDS too, issued ahead of the key stream (the waves
  // share them, each loading its part): the first key block's wait then
  // covers them, and every load in flight is of one kind, which lets the
  // compiler count them in order.
  //   q: instruction s (k-step), lane l -> head l % 32, dims kslot_dim(s, l / 32)
  //   w: lane l -> the aligned dword holding head min(l, H_I - 1)
  {
    const int hc = min(l & 31, H_I - 1);
#pragma unroll
    for (int s = wv * (KS / WPT); s < (wv + 1) * (KS / WPT); ++s)
      lds_dma16(q_idx + ((int64_t)b * H_I + hc) * DI + kslot_dim<FP8>(s, g), qw_lds + 1024 * s);
    if (wv == 0) {
      const int64_t we = (int64_t)b * w_ld + min(l, H_I - 1);
      lds_dma4(w + (we & ~(int64_t)1), qw_lds + 1024 * KS);
    }
  }

  // lane permutation of a load instruction: row l % kRowsPerKiB, chunk l / kRowsPerKiB
  const int lrow = l % St::kRowsPerKiB, lchunk = l / St::kRowsPerKiB;
  // issue the loads of stage st into its buffer (fp8: the key scales first,
  // then the rows); rows are clamped to the last visible position, so
  // nothing past the context is ever read
  auto issue = [&](int st) {
    uint8_t* buf = stage + (st % St::kBufs) * St::kBufBytes;
    if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < St::kScaleLoads; ++c) {
        const int64_t jl = min<int64_t>(jw0 + st * SROWS + 64 * c + l, p);
        lds_dma4(k_scale + row0 + jl, buf + St::kKeyBytes + 256 * c);
      }
    }
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int r = st * SROWS + c * St::kRowsPerKiB + lrow;  // row of this wave's range
      const int64_t jl = min<int64_t>(jw0 + r, p);
      lds_dma16(k_idx + (row0 + jl) * ROWB + 16 * lchunk, buf + c * St::kStride);
    }
  };
  // Every stage of the tile is loaded and scored, also past the last valid
  // key (those rows repeat it and their scores are dropped), so that the
  // pipeline and its load counts are the same for every tile.
#pragma unroll
  for (int st = 0; st < St::kBufs; ++st) issue(st);

  // Query rows and head weights: they were issued before every stage load,
  // so they have landed once no more than the stage loads are outstanding
  // (and, with several waves, once every wave got there).
  wait_vmcnt(St::kBufs * NL);
  if constexpr (WPT > 1) dma_barrier();
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 qa[KS];
  float wr[16];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qa[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qw_lds + 1024 * s + 16 * l));
  {
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(qw_lds + 1024 * KS);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hr = 8 * (r >> 2) + 4 * g + (r & 3);
      const int64_t we = (int64_t)b * w_ld + min(hr, H_I - 1);
      const uint32_t v = wl[min(hr, H_I - 1)] >> (16 * (int)(we & 1));
      wr[r] = hr < H_I ? bf16_to_f32((uint16_t)v) : 0.f;
    }
  }
  // the new key as it goes into the cache (fp8: codes + scale), landed with
  // the query rows
  [[maybe_unused]] uint32_t kcode = kpair;
  [[maybe_unused]] float ksig = 1.f;
  if constexpr (APPEND && FP8) {
    if (own) kcode = e4m3_row_pair(bf16_to_f32((uint16_t)(kpair & 0xffffu)),
                                   bf16_to_f32((uint16_t)(kpair >> 16)), &ksig);
  }

  // Score one stage.  `later` (a compile-time constant) is the number of
  // stages issued after this one that are still in flight.  Scores go to
  // the tile's LDS score buffer.
  auto do_stage = [&](int st, auto later_c) {
    constexpr int later = decltype(later_c)::value;
    const uint8_t* buf = stage + (st % St::kBufs) * St::kBufBytes;
#pragma unroll
    for (int bl = 0; bl < SBLK; ++bl) {
      // the scales and blocks 0..bl of this stage have landed once at most
      // this many loads are outstanding
      wait_vmcnt(NI - IPB * (bl + 1) + later * NL);
      // keep the scheduler from hoisting consumers of loaded registers above
      // the wait (the compiler would then wait for every load instead)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (APPEND) {
        // row p of this block (its old contents have landed): the new key
        if (own && st * SROWS + 32 * bl <= r_p && r_p < st * SROWS + 32 * bl + 32) {
          uint8_t* bufw = stage + (st % St::kBufs) * St::kBufBytes;
          const int Rp = r_p - st * SROWS;
          if (2 * l < DI) {
            if constexpr (FP8)
              *reinterpret_cast<uint16_t*>(bufw + St::offset(Rp, l >> 3) + 2 * (l & 7)) =
                  (uint16_t)kcode;
            else
              *reinterpret_cast<uint32_t*>(bufw + St::offset(Rp, l >> 2) + 4 * (l & 3)) = kcode;
          }
          if (FP8 && l == 0) *reinterpret_cast<float*>(bufw + St::kKeyBytes + 4 * Rp) = ksig;
        }
      }
      const int R = 32 * bl + (l & 31);  // stage row of this lane's key
      u32x4 kv[NLD];
#pragma unroll
      for (int c = 0; c < NLD; ++c)
        kv[c] = *reinterpret_cast<const u32x4*>(buf + St::offset(R, 2 * c + g));
      const float sig = FP8 ? *reinterpret_cast<const float*>(buf + St::kKeyBytes + 4 * R) : 1.f;
      f32x16 acc = {};
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < NLD; ++c) {
          acc = mfma32(qa[2 * c], fp8x8_to_bf16x8(kv[c][0], kv[c][1]), acc);
          acc = mfma32(qa[2 * c + 1], fp8x8_to_bf16x8(kv[c][2], kv[c][3]), acc);
        }
      } else {
#pragma unroll
        for (int c = 0; c < NLD; ++c) acc = mfma32(qa[c], as_bf16x8(kv[c]), acc);
      }
      float sl = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sl += wr[r] * relu(sig * acc[r]);
      sl = xor32_add(sl);
      // kept in LDS; global stores wait for the end: a store in flight would
      // count against the loads' waits
      if (g == 0) sc_lds[wv * TW + st * SROWS + R] = sl;
    }
  };
  // steady state: kBufs - 1 later stages in flight; the loop body is one
  // stage, so code size does not grow with the tile
  constexpr int NB = St::kBufs;
#pragma unroll 1
  for (int st = 0; st < NSTAGE - (NB - 1); ++st) {
    do_stage(st, std::integral_constant<int, NB - 1>{});
    if (st + NB < NSTAGE) {
      // every operand read of this buffer has returned (the MFMAs consumed
      // them); refill it with stage st + NB
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
      issue(st + NB);
    }
  }
  // drain: the last NB - 1 stages, with fewer and fewer later stages
  if constexpr (NB >= 4) do_stage(NSTAGE - 3, std::integral_constant<int, 2>{});
  if constexpr (NB >= 3) do_stage(NSTAGE - 2, std::integral_constant<int, 1>{});
  if constexpr (NB >= 2) do_stage(NSTAGE - 1, std::integral_constant<int, 0>{});

  // this wave's scores: coalesced stores (value i of lane l is element
  // 64 i + l of the wave's range; LDS operations of one wave run in order)
  float* const out_row = scores + (int64_t)b * ld + j0;
#pragma unroll
  for (int i = 0; i < VW; ++i) {
    const int jl = wv * TW + 64 * i + l;
    if (jl < n_valid) out_row[jl] = sc_lds[jl];
  }
  if constexpr (APPEND) {
    // every load is consumed: the new rows go into the caches
    if (own) {
      const int64_t row = row0 + p;
      if (2 * l < DI) {
        if constexpr (FP8)
          *reinterpret_cast<uint16_t*>(app.k_idx_cache + row * DI + 2 * l) = (uint16_t)kcode;
        else
          *reinterpret_cast<uint32_t*>(app.k_idx_cache + row * 2 * DI + 4 * l) = kcode;
      }
      if (FP8 && l == 0) app.k_scale_cache[row] = ksig;
      const int nc = app.D / 8;
      const bool is_v = l >= nc;
      uint16_t* dst = is_v ? app.v_cache : app.k_cache;
      const uint16_t* src = is_v ? app.v_new : app.k_new;
      if (l < 2 * nc && src != nullptr)
        *reinterpret_cast<u32x4*>(dst + row * app.D + 8 * (is_v ? l - nc : l)) = kvrow;
    }
  }
  if constexpr (REPORT) {
    const int64_t nrow = p + 1;
    if (nrow <= kDirectMax) return;  // selected straight from its scores
    if constexpr (WPT > 1) {
      dma_barrier();  // every wave's scores are in LDS
      if (wv != 0) return;
    }
    const int S = topk_subtile(nrow, topk);  // a power of two dividing TILE
    const int64_t slot = (int64_t)b * stride + (int64_t)ti * (TILE >> (31 - __clz(S)));
    if (S < TILE) {
      wave_subtile_reports<V>([&](int e) { return sc_lds[e]; }, n_valid, j0, S, hdr + slot,
                              rep_u + slot * kRep, rep_j + slot * kRep);
      return;
    }
    // report value i of lane l is tile element V l + i
    uint32_t uv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) uv[i] = order_key(sc_lds[V * l + i]);
    wave_tile_report<V>(uv, min(max(n_valid - V * l, 0), V), j0 + V * l, hdr + slot,
                        rep_u + slot * kRep, rep_j + slot * kRep);
  }
}

// waves per tile of the deep pipeline
constexpr int kDeepWaves(int tile) { return tile == 256 ? 4 : (tile >= 128 ? 2 : 1); }

template <int DI, bool FP8, bool REPORT, bool APPEND>
static hipError_t launch_decode_tiled(int tile, const uint16_t* q, const uint16_t* w,
                                      int64_t w_ld, const uint8_t* k, const float* ks, int H_I,
                                      const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                      int max_ctx, float* scores, int64_t ld, RepHeader* hdr,
                                      uint32_t* ru, int32_t* rj, int stride, int topk,
                                      const DecodeAppend& app, hipStream_t st, hipEvent_t ev0,
                                      hipEvent_t ev1) {
  dim3 grid((max_ctx + tile - 1) / tile, B);
  // Few tiles per CU (256 CUs): several waves per tile, each with a deep
  // pipeline, so more loads are in flight per CU (256-key tiles: four waves
  // of 64 keys, measured 0.7 us faster per 128K decode step than two of
  // 128); many tiles: one wave per tile with a shallow pipeline, so more
  // waves fit in LDS.
  const bool deep = (int64_t)grid.x * B <= 1024;
  // with events: the dispatch itself records them at the kernel's start and end
#define DSA_DECODE_LAUNCH(KER, NT)                                                             \
  if (ev0)                                                                                     \
    hipExtLaunchKernelGGL(KER, grid, dim3(NT), 0, st, ev0, ev1, 0, q, w, w_ld, k, ks, H_I,     \
                          ctx_len, cu_ctx, scores, ld, hdr, ru, rj, stride, topk, app);        \
  else                                                                                         \
    hipLaunchKernelGGL(KER, grid, dim3(NT), 0, st, q, w, w_ld, k, ks, H_I, ctx_len, cu_ctx,    \
                       scores, ld, hdr, ru, rj, stride, topk, app);
#define DSA_DECODE_TILE(T_)                                                                    \
  case T_:                                                                                     \
    if (deep) {                                                                                \
      DSA_DECODE_LAUNCH((index_decode_kernel<DI, FP8, T_, REPORT, true, kDeepWaves(T_), APPEND>), \
                        64 * kDeepWaves(T_))                                              \
    } else {                                                                                   \
      DSA_DECODE_LAUNCH((index_decode_kernel<DI, FP8, T_, REPORT, false, 1, APPEND>), 64)      \
    }                                                                                          \
    break;
  switch (tile) {
    DSA_DECODE_TILE(64)
    DSA_DECODE_TILE(128)
    DSA_DECODE_TILE(256)
    DSA_DECODE_TILE(512)
    DSA_DECODE_TILE(1024)
    DSA_DECODE_TILE(2048)
    default:
      return hipErrorInvalidValue;
  }
#undef DSA_DECODE_TILE
#undef DSA_DECODE_LAUNCH
  return hipGetLastError();
}

template <int DI, bool FP8>
static hipError_t launch_decode_any(bool report, int tile, const uint16_t* q, const uint16_t* w,
                                    int64_t w_ld, const uint8_t* k, const float* ks, int H_I,
                                    const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                    int max_ctx, float* scores, int64_t ld, RepHeader* hdr,
                                    uint32_t* ru, int32_t* rj, int stride, int topk,
                                    const DecodeAppend* app, hipStream_t st, hipEvent_t ev0,
                                    hipEvent_t ev1) {
  const DecodeAppend none = {};
#define DSA_DECODE_ANY(R_, A_)                                                                 \
  return launch_decode_tiled<DI, FP8, R_, A_>(tile, q, w, w_ld, k, ks, H_I, ctx_len, cu_ctx, B, \
                                              max_ctx, scores, ld, hdr, ru, rj, stride, topk,  \
                                              app ? *app : none, st, ev0, ev1)
  if (report) {
    if (app) DSA_DECODE_ANY(true, true);
    DSA_DECODE_ANY(true, false);
  }
  if (app) DSA_DECODE_ANY(false, true);
  DSA_DECODE_ANY(false, false);
#undef DSA_DECODE_ANY
}

hipError_t launch_index_decode(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                               int k_dtype, const float* k_scale, int H_I, int d_I,
                               const int32_t* ctx_len, const int64_t* cu_ctx, int B, int max_ctx,
                               float* scores, int64_t ld, const TopkWs* reports,
                               const DecodeAppend* app, hipStream_t stream, hipEvent_t ev0,
                               hipEvent_t ev1) {
  const int tile = reports ? reports->tile : 256;
  RepHeader* hdr = reports ? reports->hdr : nullptr;
  uint32_t* ru = reports ? reports->rep_u : nullptr;
  int32_t* rj = reports ? reports->rep_j : nullptr;
  const int ntm = reports ? reports->stride : 0;
  const int topk = reports ? reports->K : 0;
  auto q = static_cast<const uint16_t*>(q_idx);
  auto wp = static_cast<const uint16_t*>(w);
  auto k = static_cast<const uint8_t*>(k_idx);
  const bool fp8 = k_dtype == 1;
  const bool rep = reports != nullptr;
  if (d_I == 128 && !fp8)
    return launch_decode_any<128, false>(rep, tile, q, wp, w_ld, k, k_scale, H_I, ctx_len,
                                         cu_ctx, B, max_ctx, scores, ld, hdr, ru, rj, ntm, topk, app, stream, ev0, ev1);
  if (d_I == 128 && fp8)
    return launch_decode_any<128, true>(rep, tile, q, wp, w_ld, k, k_scale, H_I, ctx_len, cu_ctx,
                                        B, max_ctx, scores, ld, hdr, ru, rj, ntm, topk, app, stream, ev0, ev1);
  if (d_I == 64 && !fp8)
    return launch_decode_any<64, false>(rep, tile, q, wp, w_ld, k, k_scale, H_I, ctx_len, cu_ctx,
                                        B, max_ctx, scores, ld, hdr, ru, rj, ntm, topk, app, stream, ev0, ev1);
  if (d_I == 64 && fp8)
    return launch_decode_any<64, true>(rep, tile, q, wp, w_ld, k, k_scale, H_I, ctx_len, cu_ctx,
                                       B, max_ctx, scores, ld, hdr, ru, rj, ntm, topk, app, stream, ev0, ev1);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------
// Row i of a 32-row MFMA block <-> (query within block, head).  Chosen so
// that the 16 accumulator rows of each lane are whole queries.
template <int HI>
struct RowMap {
  static constexpr int QPB = 32 / HI;  // queries per 32-row block
  __device__ static int query_of_row(int i) {
    return HI == 4 ? (i >> 2) : (HI == 16 ? ((i >> 2) & 1) : 0);
  }
  __device__ static int head_of_row(int i) {
    return HI == 4 ? (i & 3) : (HI == 16 ? (4 * (i >> 3) + (i & 3)) : i);
  }
};

// Prefill workgroup = NCW compute waves + one loader wave, or (SELF) NCW
// compute waves that load the stages themselves.
//   - the loader streams the key range in stages of KT keys into a ring of
//     NBUF LDS buffers with direct global-to-LDS loads; its load counter
//     tracks nothing else, so its waits are exact.  In the SELF form every
//     compute wave issues its share of each stage's load instructions right
//     after the stage barrier and waits for all of its memory operations
//     (vmcnt(0)) before the next one; its score stores are kept back in a
//     per-wave LDS stash and go out during the next stage's first two
//     blocks, so that wait finds them long done.  (Flushing the stash right
//     after the barrier, with every wave at once, idled the matrix pipes
//     and made the kernel 6% slower than the loader form.)  Two buffers of 128 keys
//     (256 with fp8 query heads, whose operands take fewer registers)
//     measured 4-7% faster than four of 64: half the workgroup barriers per
//     key, and the same bytes in flight;
//   - the compute waves hold their query heads (A operand, MB blocks of 32
//     (query, head) rows) in registers, run the MFMAs on the stage's keys,
//     apply ReLU / head weights / head sum in registers and store the
//     stage's scores (causal positions only) straight from registers; they
//     never wait on their stores.  Inside a wave the stage's 32-key blocks
//     form a pipeline: the MFMAs of one block run while the wave reduces
//     the previous block (vector ALU) and reads the next block's B operands
//     from LDS, so the wave keeps its own matrix pipe busy through its
//     epilogues.
// One workgroup barrier per stage orders the two roles; it waits for no
// memory traffic (the loader waits for its stages explicitly).
template <int DI, int HI, bool FP8, int KT_>
struct PrefillShape {
  static constexpr int KT = KT_;                         // keys per stage
  static constexpr int ROWB = FP8 ? DI : 2 * DI;         // bytes per key row
  static constexpr int SB = KT * ROWB;                   // key bytes per stage
  static constexpr int RPK = 1024 / ROWB;                // rows per 1 KiB load
  static constexpr int PAD = RPK >= 16 ? 0 : 256 / RPK;  // LDS pad per KiB
  static constexpr int STRIDE = 1024 + PAD;
  static constexpr int NI = SB / 1024;                   // key loads per stage
  static constexpr int NL = NI + (FP8 ? KT / 64 : 0);    // all loads per stage
  static constexpr int KEYB = NI * STRIDE;
  static constexpr int BUFB = KEYB + (FP8 ? 4 * KT : 0); // LDS bytes per stage buffer
  __device__ static int offset(int r, int ck) {
    return (r / RPK) * STRIDE + (ck * RPK + r % RPK) * 16;
  }
};

// Q8 (fp8 keys only): the query heads are E4M3FN codes with one fp32 scale
// per (query, head), and the contraction runs on the fp8 MFMA
// (v_mfma_f32_32x32x64_f8f6f4, two k-steps of 64 dims at d_I = 128).  Its
// operands are 32 bytes per lane: row / column l % 32, k slots 32 (l / 32)
// + e (checked on the GPU); k-step s of lane half g takes the key row's
// 16-byte chunks 4 s + g and 4 s + 2 + g (the chunks the fp8-key B reads
// already fetch) and the query row's same bytes.  With positive scales
// (the quantiser's amax / 448) the epilogue folds the query scale into the
// head weight and applies the key scale once per key after the head sum:
// s = sigma_j * sum_h (w_h rho_h) ReLU(acc_h).
template <int DI, int HI, bool FP8, int MB, int NCW, int NBUF, bool Q8, bool SELF>
__global__ __launch_bounds__(64 * (NCW + (SELF ? 0 : 1))) void index_prefill_kernel(
    const void* __restrict__ q_idx_v, const float* __restrict__ q_scale,
    const uint16_t* __restrict__ w, int64_t w_ld, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ k_scale, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ ctx_len, const int64_t* __restrict__ cu_ctx,
    float* __restrict__ scores, int64_t ld, int nsplit, int qtiles, int nitems) {
  static_assert(!Q8 || FP8, "fp8 query heads need fp8 keys");
  const uint16_t* __restrict__ q_idx = static_cast<const uint16_t*>(q_idx_v);
  const uint8_t* __restrict__ q8 = static_cast<const uint8_t*>(q_idx_v);
  using PS = PrefillShape<DI, HI, FP8, Q8 ? 256 : 128>;
  constexpr int KT = PS::KT;
  constexpr int KS = DI / 16;
  constexpr int ROWB = PS::ROWB;
  constexpr int QPB = RowMap<HI>::QPB;
  constexpr int QW = MB * QPB;               // queries per compute wave
  constexpr int QWG = NCW * QW;              // queries per workgroup
  constexpr int NLD = FP8 ? KS / 2 : KS;     // 16-byte operand chunks per lane per key block
  static_assert(PS::NL * (NBUF - 1) <= 63, "loads in flight");

  constexpr int NB = KT / 32;                // 32-key blocks per stage
  constexpr int NSUM = HI == 4 ? 4 : 1;      // sums per query block per lane
  // SELF: per wave, the sums of the blocks reduced during one stage, stored
  // to memory during the next stage's first two blocks
  constexpr int kStash = SELF ? NB * MB * NSUM * 64 * 4 : 0;
  __shared__ __attribute__((aligned(16))) uint8_t lds[NBUF * PS::BUFB + NCW * kStash];
  uint8_t* const ring = lds;

  // Work item of this workgroup.  Workgroups go to the 8 XCDs in turn
  // (id % 8); XCD x takes the contiguous run of items [x n8, (x + 1) n8),
  // ordered sequence-major, then split, then query tile, so the workgroups
  // an XCD runs at one time mostly stream the same key range through its L2.
  const int n8 = (nitems + 7) >> 3;
  const int item = (int)(blockIdx.x & 7) * n8 + (int)(blockIdx.x >> 3);
  if (item >= nitems) return;
  const int per_b = nsplit * qtiles;
  const int b = item / per_b, split = (item - b * per_b) / qtiles;
  const int qt = item - b * per_b - split * qtiles;
  const int nq = cu_q[b + 1] - cu_q[b];
  const int qbase = qt * QWG;
  if (qbase >= nq) return;
  const int64_t L = ctx_len[b];
  const int64_t pos0 = L - nq;               // position of query 0 of the sequence
  const int64_t row0 = cu_ctx[b];
  const int64_t t0 = cu_q[b];
  const int l = lane_id(), g = l >> 5, wv = wave_id();
  // visible key range of this workgroup: [0, last position of its queries]
  const int qlast = min(nq, qbase + QWG) - 1;
  const int64_t kend = pos0 + qlast + 1;
  const int64_t nst_all = (kend + KT - 1) / KT;
  const int64_t st_lo = nst_all * split / nsplit;
  const int nst = (int)(nst_all * (split + 1) / nsplit - st_lo);
  if (nst <= 0) return;

  if (!SELF && wv == NCW) {
    // ---------------- loader ----------------
    const int lrow = l % PS::RPK, lchunk = l / PS::RPK;
    auto issue = [&](int k) {
      uint8_t* buf = ring + (k % NBUF) * PS::BUFB;
      const int64_t kb = (st_lo + k) * KT;
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < KT / 64; ++c)
          lds_dma4(k_scale + row0 + min<int64_t>(kb + 64 * c + l, L - 1), buf + PS::KEYB + 256 * c);
      }
#pragma unroll
      for (int c = 0; c < PS::NI; ++c)
        lds_dma16(k_idx + (row0 + min<int64_t>(kb + c * PS::RPK + lrow, L - 1)) * ROWB +
                      16 * lchunk,
                  buf + c * PS::STRIDE);
    };
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (k < nst) issue(k);
#pragma unroll 1
    for (int i = 0; i < nst; ++i) {
      // stage i has landed once only the stages issued after it are in flight
      const int later = min(NBUF - 2, nst - 1 - i);
      wait_vmcnt(later * PS::NL);
      dma_barrier();
      if (i + NBUF - 1 < nst) issue(i + NBUF - 1);  // into the buffer of stage i - 1
    }
    return;
  }
  // ---------------- compute waves ----------------
  const int wq0 = qbase + wv * QW;
  constexpr int KS8 = DI / 64;  // fp8 MFMA k-steps
  bf16x8 qa[Q8 ? 1 : MB][Q8 ? 1 : KS];
  v8i32 qa8[Q8 ? MB : 1][Q8 ? KS8 : 1];
  float wr[MB][16];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int i = l & 31;
    const int qq = min(wq0 + m * QPB + RowMap<HI>::query_of_row(i), nq - 1);
    const int hh = RowMap<HI>::head_of_row(i);
    if constexpr (Q8) {
      const uint8_t* qr = q8 + ((t0 + qq) * HI + hh) * DI;
#pragma unroll
      for (int s = 0; s < KS8; ++s) {
        const u32x4 lo = ld16(qr + 16 * (4 * s + g)), hi = ld16(qr + 16 * (4 * s + 2 + g));
        qa8[m][s] = v8i32{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qa[m][s] = as_bf16x8(ld16(q_idx + ((t0 + qq) * HI + hh) * DI + kslot_dim<FP8>(s, g)));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = 8 * (r >> 2) + 4 * g + (r & 3);
      const int q2 = wq0 + m * QPB + RowMap<HI>::query_of_row(ir);
      const int64_t qrow = t0 + min(q2, nq - 1);
      const int head = RowMap<HI>::head_of_row(ir);
      float wv2 = bf16_to_f32(w[qrow * w_ld + head]);
      if constexpr (Q8) wv2 *= q_scale[qrow * HI + head];
      wr[m][r] = q2 < nq ? wv2 : 0.f;
    }
  }
  // The 32-key blocks form a pipeline inside each wave: while the MFMAs of
  // one block run, the wave reduces the previous block (ReLU, head weights,
  // head sum: vector ALU work that does not depend on those MFMAs) and
  // stores its scores.  acc[p] holds the block of parity p.
  static_assert(NB % 2 == 0, "block parity = block index within the stage, mod 2");
  f32x16 acc[2][MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[1][m] = f32x16{};
  auto reduce = [&](int p, float sgp, float (&sum)[MB][NSUM]) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int c4 = 0; c4 < NSUM; ++c4) {
        constexpr int RN = 16 / NSUM;  // heads per sum
        float s0 = 0.f, s1 = 0.f;
        if constexpr (Q8) {
#pragma unroll
          for (int r = 0; r < RN; r += 2) {
            s0 += wr[m][RN * c4 + r] * relu(acc[p][m][RN * c4 + r]);
            s1 += wr[m][RN * c4 + r + 1] * relu(acc[p][m][RN * c4 + r + 1]);
          }
          sum[m][c4] = sgp * (s0 + s1);
        } else {
#pragma unroll
          for (int r = 0; r < RN; r += 2) {
            s0 += wr[m][RN * c4 + r] * relu(sgp * acc[p][m][RN * c4 + r]);
            s1 += wr[m][RN * c4 + r + 1] * relu(sgp * acc[p][m][RN * c4 + r + 1]);
          }
          sum[m][c4] = s0 + s1;
        }
      }
  };
  // causal store of a block's scores (lanes of a half-wave: 32 consecutive
  // keys of one query); the chunk's score array is far larger than the
  // caches, so the stores carry the nontemporal hint (measured 0.6% faster
  // at 8192 queries x 139264 keys)
  auto put = [&](int q, int64_t j, float v) {  // q: query of the sequence
    if (q < nq && j <= pos0 + q) __builtin_nontemporal_store(v, &scores[(t0 + q) * ld + j]);
  };
  auto store = [&](int64_t j, const float (&sum)[MB][NSUM]) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int q0 = wq0 + m * QPB;  // first query of block m
      if constexpr (HI == 4) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) put(q0 + 2 * c4 + g, j, sum[m][c4]);
      } else if constexpr (HI == 32) {
        const float v = xor32_add(sum[m][0]);
        if (g == 0) put(q0, j, v);
      } else {
        put(q0 + g, j, sum[m][0]);
      }
    }
  };
  // SELF: wave w issues load instructions c = w, w + NCW, ... of every
  // stage (the loader's stage layout)
  [[maybe_unused]] const int wvu = __builtin_amdgcn_readfirstlane(wv);
  [[maybe_unused]] float* const stash =
      reinterpret_cast<float*>(lds + NBUF * PS::BUFB + wvu * kStash);
  [[maybe_unused]] auto issue_share = [&](int k) {
    uint8_t* buf = ring + (k % NBUF) * PS::BUFB;
    const int64_t kb = (st_lo + k) * KT;
    const int lrow = l % PS::RPK, lchunk = l / PS::RPK;
#pragma unroll
    for (int k8 = 0; k8 < (PS::NL + NCW - 1) / NCW; ++k8) {
      const int c = wvu + NCW * k8;  // wave-uniform
      if (PS::NL % NCW != 0 && c >= PS::NL) break;
      if (FP8 && c >= PS::NI)
        lds_dma4(k_scale + row0 + min<int64_t>(kb + 64 * (c - PS::NI) + l, L - 1),
                 buf + PS::KEYB + 256 * (c - PS::NI));
      else
        lds_dma16(k_idx + (row0 + min<int64_t>(kb + c * PS::RPK + lrow, L - 1)) * ROWB +
                      16 * lchunk,
                  buf + c * PS::STRIDE);
    }
  };
  // stash slot n of a stage holds the sums reduced during its block n (those
  // of the block before; the previous stage's last block for n = 0)
  [[maybe_unused]] auto stash_put = [&](int n, const float (&sum)[MB][NSUM]) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int c4 = 0; c4 < NSUM; ++c4) stash[((n * MB + m) * NSUM + c4) * 64 + l] = sum[m][c4];
  };
  // stores of slot n of stage s's stash (slot 0 of stage 0 holds nothing)
  [[maybe_unused]] auto flush = [&](int s, int n) {
    if (s == 0 && n == 0) return;
    float sum[MB][NSUM];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int c4 = 0; c4 < NSUM; ++c4) sum[m][c4] = stash[((n * MB + m) * NSUM + c4) * 64 + l];
    store((st_lo + s) * KT + 32 * (n - 1) + (l & 31), sum);
  };
  int64_t j_prev = 0;  // key of this lane in the block awaiting its reduction
  float sg_prev = 1.f;
  if constexpr (SELF) issue_share(0);
#pragma unroll 1
  for (int i = 0; i < nst; ++i) {
    // SELF: this wave's loads of stage i have landed, and its stores, issued
    // in the first half of stage i - 1, are done
    if constexpr (SELF) wait_vmcnt(0);
    dma_barrier();  // stage i has landed; every wave is done with stage i - 1
    if constexpr (SELF) {
      if (i + 1 < nst) issue_share(i + 1);  // into the buffer of stage i - 1
    }
    const uint8_t* buf = ring + (i % NBUF) * PS::BUFB;
    const int64_t kb = (st_lo + i) * KT;
    // B operands: block n + 1's reads are issued at block n's start and land
    // during its MFMAs (two blocks' operands in registers at a time)
    u32x4 kvc[NLD], kvn[NLD];
    float sgc = 1.f, sgnx = 1.f;
    auto readB = [&](int n, u32x4 (&kv)[NLD], float& sg) {
      const int R = 32 * n + (l & 31);
#pragma unroll
      for (int c = 0; c < NLD; ++c)
        kv[c] = *reinterpret_cast<const u32x4*>(buf + PS::offset(R, 2 * c + g));
      sg = FP8 ? reinterpret_cast<const float*>(buf + PS::KEYB)[R] : 1.f;
    };
    readB(0, kvc, sgc);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int R = 32 * n + (l & 31);
      if (n + 1 < NB) readB(n + 1, kvn, sgnx);
      const u32x4(&kv)[NLD] = kvc;
      const float sgn = sgc;
      const int pn = n & 1;
      // a wave in its MFMA + reduction block takes issue priority over one
      // at its stores or stage wait (same-box A/B: indexer 3871 / 3886 ->
      // 3862 / 3860 us with bf16 query heads, 2465 / 2451 -> 2430 / 2435 us
      // with fp8 ones)
      __builtin_amdgcn_s_setprio(1);
      // MFMAs of this block (the first k-step from a zero accumulator)
      if constexpr (Q8) {
#pragma unroll
        for (int s8 = 0; s8 < KS8; ++s8) {
          const u32x4 lo = kv[2 * s8], hi = kv[2 * s8 + 1];
          const v8i32 b8 = v8i32{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
          for (int m = 0; m < MB; ++m)
            acc[pn][m] = mfma_f8(qa8[m][s8], b8, s8 == 0 ? f32x16{} : acc[pn][m]);
        }
      }
#pragma unroll
      for (int c = 0; c < (Q8 ? 0 : NLD); ++c) {
        if constexpr (FP8) {
          const bf16x8 b0 = fp8x8_to_bf16x8(kv[c][0], kv[c][1]);
          const bf16x8 b1 = fp8x8_to_bf16x8(kv[c][2], kv[c][3]);
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            acc[pn][m] = mfma32(qa[m][2 * c], b0, c == 0 ? f32x16{} : acc[pn][m]);
            acc[pn][m] = mfma32(qa[m][2 * c + 1], b1, acc[pn][m]);
          }
        } else {
#pragma unroll
          for (int m = 0; m < MB; ++m)
            acc[pn][m] = mfma32(qa[m][c], as_bf16x8(kv[c]), c == 0 ? f32x16{} : acc[pn][m]);
        }
      }
      // ... and the reduction of the previous block, meanwhile (its result
      // is dropped for the very first block)
      float sum[MB][NSUM];
      reduce(pn ^ 1, sg_prev, sum);
      // issue order: the next block's B reads, then each MFMA followed by a
      // few of the reduction's vector instructions
      if (n + 1 < NB) __builtin_amdgcn_sched_group_barrier(0x100, NLD, 0);
#pragma unroll
      for (int k = 0; k < (Q8 ? KS8 : KS) * MB; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, Q8 ? 18 : 5, 0);
      }
      // the sums exist here, not only inside the stores' branches
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int c4 = 0; c4 < NSUM; ++c4) asm volatile("" : "+v"(sum[m][c4]));
      if constexpr (SELF) {
        // the previous stage's slots go out during blocks 0 and 1, each slot
        // before this stage overwrites it
        constexpr int HALF = NB / 2;
        if (i > 0 && n < 2) {
#pragma unroll
          for (int h = 0; h < HALF; ++h) flush(i - 1, n * HALF + h);
        }
        stash_put(n, sum);
      } else if (i > 0 || n > 0) {
        store(j_prev, sum);
      }
      __builtin_amdgcn_s_setprio(0);
      j_prev = kb + R;
      sg_prev = sgn;
      if (n + 1 < NB) {
#pragma unroll
        for (int c = 0; c < NLD; ++c) kvc[c] = kvn[c];
        sgc = sgnx;
      }
    }
  }
  if constexpr (SELF) {
    for (int n = 0; n < NB; ++n) flush(nst - 1, n);
  }
  {
    float sum[MB][NSUM];
    reduce((NB - 1) & 1, sg_prev, sum);
    store(j_prev, sum);
  }
}

// Workgroups of `kernel` (block of `threads`) resident on the whole device
// at once: CUs x workgroups per CU (from the occupancy calculator), looked
// up once per device and kernel.
static int prefill_slots(const void* kernel, int threads) {
  struct Entry {
    int dev;
    const void* k;
    int slots;
  };
  static Entry cache[16];
  static int ncache = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < ncache; ++i)
    if (cache[i].dev == dev && cache[i].k == kernel) return cache[i].slots;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int slots = cus * per_cu;
  if (ncache < 16) cache[ncache++] = Entry{dev, kernel, slots};
  return slots;
}

template <int DI, int HI, bool FP8, bool Q8, int NCW, bool SELF>
static hipError_t launch_prefill_v(const void* q, const float* qs, const uint16_t* w, int64_t w_ld,
                                   const uint8_t* k, const float* ks, const int32_t* cu_q,
                                   const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                   int max_q, int max_ctx, float* scores, int64_t ld,
                                   hipStream_t st) {
  // eight waves per workgroup (two per SIMD at this register use): NCW = 7
  // compute waves + the loader, or 8 self-loading compute waves; two 32-row
  // query blocks per compute wave where the registers allow it (8 queries
  // of 4 heads fill a block)
  constexpr int MB = HI == 4 ? 1 : 2, NBUF = 2;
  constexpr int NT = 64 * (NCW + (SELF ? 0 : 1));
  constexpr int QWG = NCW * MB * (32 / HI);
  const int qtiles = (max_q + QWG - 1) / QWG;
  // Enough workgroups to fill the chip: the key range of each query tile is
  // split when the tiles alone are too few.  The workgroups run in rounds
  // of `slots` (CUs x resident workgroups per CU) and take about equally
  // long, so among the split counts that give 4 to 8 rounds (or, when even
  // 4 rounds are out of reach, any count) the one that leaves the least of
  // the last round idle is taken (e.g. 8192 queries of 16 heads in 28-query
  // tiles: 293 tiles, 6 splits = 1758 workgroups = 6.9 rounds of 256, where
  // 4 splits gave 4.6 rounds; in 32-query tiles: 256 x 4 = 4.0 rounds).  Each split keeps at least 4096 keys, so that loading
  // the query heads and filling the stage ring stay a small part of it.
  auto ker = index_prefill_kernel<DI, HI, FP8, MB, NCW, NBUF, Q8, SELF>;
  const int slots = prefill_slots(reinterpret_cast<const void*>(ker), NT);
  const int64_t tiles = (int64_t)qtiles * B;
  int nsplit = 1;
  if (tiles < 4 * (int64_t)slots) {
    const int nmax = std::max(1, std::min(64, max_ctx / 4096));
    const bool reach4 = tiles * nmax >= 4 * (int64_t)slots;
    double best = 1e30;
    for (int n = 1; n <= nmax; ++n) {
      const int64_t wgs = tiles * n;
      if (reach4 && wgs < 4 * (int64_t)slots) continue;
      if (reach4 && wgs > 8 * (int64_t)slots) break;
      const double rounds = (double)wgs / slots;
      const double waste = std::ceil(rounds) / rounds;  // time over the ideal time
      if (waste < best - 1e-3) {
        best = waste;
        nsplit = n;
      }
    }
  }
  const int64_t nitems = tiles * nsplit;
  if (nitems > (int64_t)INT32_MAX - 8) return hipErrorInvalidValue;
  const int grid = (int)((nitems + 7) / 8) * 8;
  hipLaunchKernelGGL(ker, dim3(grid), dim3(NT), 0, st, q, qs, w, w_ld, k, ks, cu_q,
                     ctx_len, cu_ctx, scores, ld, nsplit, qtiles, (int)nitems);
  return hipGetLastError();
}

template <int DI, int HI, bool FP8, bool Q8>
static hipError_t launch_prefill_t(const void* q, const float* qs, const uint16_t* w, int64_t w_ld,
                                   const uint8_t* k, const float* ks, const int32_t* cu_q,
                                   const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                   int max_q, int max_ctx, float* scores, int64_t ld,
                                   hipStream_t st) {
  // bf16 keys: 8 compute waves that load their own stages (1% faster at
  // 8192 queries x 139264 keys than 7 + a loader wave); fp8 keys, whose
  // epilogue and operand conversions keep the vector ALU busy, stay with
  // the loader wave (the self-loading form is 6% slower there)
  if constexpr (FP8)
    return launch_prefill_v<DI, HI, FP8, Q8, 7, false>(q, qs, w, w_ld, k, ks, cu_q, ctx_len,
                                                       cu_ctx, B, max_q, max_ctx, scores, ld, st);
  else
    return launch_prefill_v<DI, HI, FP8, Q8, 8, true>(q, qs, w, w_ld, k, ks, cu_q, ctx_len,
                                                      cu_ctx, B, max_q, max_ctx, scores, ld, st);
}

hipError_t launch_index_prefill(const void* q_idx, int q_dtype, const float* q_scale,
                                const void* w, int64_t w_ld, const void* k_idx, int k_dtype,
                                const float* k_scale, int H_I, int d_I, const int32_t* cu_q,
                                const int32_t* ctx_len, const int64_t* cu_ctx, int B, int max_q,
                                int max_ctx, float* scores, int64_t ld, hipStream_t stream) {
  auto wp = static_cast<const uint16_t*>(w);
  auto k = static_cast<const uint8_t*>(k_idx);
  const bool fp8 = k_dtype == 1, q8 = q_dtype == 1;
  if (q8 && !fp8) return hipErrorInvalidValue;
#define DSA_PREFILL_CASE(DI_, HI_)                                                              \
  if (d_I == DI_ && H_I == HI_) {                                                               \
    if (q8)                                                                                     \
      return launch_prefill_t<DI_, HI_, true, true>(q_idx, q_scale, wp, w_ld, k, k_scale, cu_q, \
                                                    ctx_len, cu_ctx, B, max_q, max_ctx, scores, \
                                                    ld, stream);                                \
    return fp8 ? launch_prefill_t<DI_, HI_, true, false>(q_idx, nullptr, wp, w_ld, k, k_scale,  \
                                                         cu_q, ctx_len, cu_ctx, B, max_q,      \
                                                         max_ctx, scores, ld, stream)          \
               : launch_prefill_t<DI_, HI_, false, false>(q_idx, nullptr, wp, w_ld, k, k_scale, \
                                                          cu_q, ctx_len, cu_ctx, B, max_q,     \
                                                          max_ctx, scores, ld, stream);        \
  }
  DSA_PREFILL_CASE(128, 32)
  DSA_PREFILL_CASE(128, 16)
  DSA_PREFILL_CASE(64, 4)
#undef DSA_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
