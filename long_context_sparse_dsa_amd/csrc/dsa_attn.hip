// dsa_attn.hip -- gated sparse attention over gathered K/V rows.
//
// For query row t and head h, over the selected positions S (one index row
// per query shared by every head; one shared K/V head):
//   o = softmax_{j in S}(c * q[t,h,:] . K[j,:]) @ V[S,:],  out = o * sigmoid(g)
// ("Open-Source LLM Architecture Evolution ...", Technical Deep Dive item 2:
// scores and softmax over only the selected 2048; Architecture Breakdown
// item 2 and the deployment page section 2: gated layers.)  With idx == NULL
// the set is the sliding window {p-W+1 .. p} (the naive-n0-5-flash page).
//
// Kernel layout (gfx950, wave64, 4 waves per workgroup):
//   - a workgroup takes `rows_per_split` consecutive entries of the query's
//     index row (staged in LDS first) in steps of 32 RB rows; wave
//     (rb, hb) takes rows 32 rb .. 32 rb + 31 of a step for heads
//     32 hb .. 32 hb + 31 and keeps its own running softmax state (max, sum,
//     O^T accumulators); the row-block states are merged through LDS at the
//     end;
//   - each K and V row of a step is gathered once per workgroup: one wave
//     of a row block loads its K rows, the other its V rows, a step ahead,
//     into registers (four whole rows per load instruction); at the step's
//     start they go to double-buffered, XOR-swizzled LDS tiles that both
//     head blocks read (RowTile);
//   - S^T = K_rows . q^T on MFMA (v_mfma_f32_32x32x16_bf16): the A operand
//     comes from the K tile, q is the B operand, held in registers for the
//     whole kernel;
//   - in the S^T accumulator layout each lane holds one head and 16 rows, so
//     the per-head max / sum need one cross-half exchange, and P^T is
//     already a B operand once its k slots are taken in accumulator order;
//     the reference max moves only when a head's step max passes it by a
//     margin, so most steps leave O unscaled;
//   - the A operand of O^T = V^T . P^T (8 rows of one dim per lane) comes
//     from the V tile with the LDS transpose read ds_read_b64_tr_b16, whose
//     16-lane groups turn 4 rows x 16 dims into 16 dims x 4 rows;
//   - with several splits per query the workgroups write partial (m, l, O)
//     and a combine kernel merges them and applies the gate.
#include <type_traits>

#include "dsa_kernels.h"
#include "dsa_device.h"
#include "dsa_attn_tile.h"

namespace dsa {

// Index rows a workgroup stages in LDS (index mode); longer lists are split.
constexpr int kAttnMaxRows = 2048;
// The online softmax moves its reference max only past this margin (log2).
constexpr float kRescale = 8.f;

template <int D, int HB, bool FINAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ idx, int K, int window,
    const uint16_t* __restrict__ gate, int gstride, float scale_log2, int Hq, const int32_t* cu_q,
    const int32_t* ctx_len, const int64_t* cu_ctx, int B, int rows_per_split,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part, int nsplit,
    AttnLayers layers) {
  if (layers.n > 0) {  // one of several layers (grid z), each with its own tensors
    const int z = blockIdx.z;
    q = layers.q[z];
    kc = layers.kc[z];
    vc = layers.vc[z];
    gate = layers.gate[z];
    out = layers.out[z];
  }
  constexpr int KS = D / 16;   // k-steps of q . K
  constexpr int DB = D / 32;   // 32-wide blocks of the output dim
  constexpr int RB = 4 / HB;   // row-block waves per head block
  constexpr int STEP = 32 * RB;  // rows per workgroup step
  using VT = RowTile<D>;
  // merge state of one wave: per lane (m, l) and DB x 16 O values
  constexpr int ST_FLOATS = 2 + DB * 16;
  constexpr int MERGE_BYTES = (RB / 2) * HB * 64 * ST_FLOATS * 4;
  constexpr int TILE_BYTES = 2 * RB * 2 * VT::kBytes;  // 2 buffers x RB row blocks x {K, V}
  constexpr int SMEM_BYTES = MERGE_BYTES > TILE_BYTES ? MERGE_BYTES : TILE_BYTES;
  // One LDS array: the staged index entries (index mode) first, so that
  // the step loop's reads of them take immediate offsets, then the tiles
  // (and the merge area over them).
  constexpr int kIdxPad = 2 * STEP;
  constexpr int IDX_BYTES = (kAttnMaxRows + kIdxPad) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[IDX_BYTES + SMEM_BYTES];
  int32_t* const idx_lds = reinterpret_cast<int32_t*>(lds_all);
  uint8_t* const smem = lds_all + IDX_BYTES;

  // Workgroups go to the 8 XCDs (each with its own L2) in turn.  With one
  // workgroup per query, query t + 1 would land on another XCD than query t,
  // though neighbouring queries select mostly the same K/V rows; instead
  // each XCD takes a contiguous run of queries.
  int t = blockIdx.y;
  if (gridDim.x == 1) {
    const int T = gridDim.y, x = t & 7, i = t >> 3, q = T >> 3, r = T & 7;
    t = x * q + min(x, r) + i;
  }
  const int split = blockIdx.x;
  const int l = lane_id(), g = l >> 5, wv = wave_id();
  const int hb = wv % HB, rb = wv / HB;
  const int lo = split * rows_per_split;
  // index-list entry of this lane's row in step i: lp0 + STEP i
  const int lp0 = lo + 32 * rb + (l & 31);
  // In index mode the workgroup's part of the index row (at most
  // kAttnMaxRows entries) goes to LDS first; these loads do not depend on
  // the batch descriptor, so they share its round trip.  Each entry is
  // checked once as it is staged: entries past the list, and entries
  // outside [0, p] (the -1 padding, or anything else a caller passed), are
  // staged as -1.  The array runs two steps past kAttnMaxRows (staged -1),
  // so the step loop reads it unclamped.
  constexpr int PT = kAttnMaxRows / 256;
  int32_t iv[PT];
  if (idx) {
    const int nr = min(K, lo + rows_per_split) - lo;
    const int32_t* src = idx + (int64_t)t * K + lo;
#pragma unroll
    for (int r = 0; r < PT; ++r) {
      const int e = (int)threadIdx.x + 256 * r;
      iv[r] = e < nr ? src[e] : -1;
    }
  }
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t row0 = cu_ctx[ri.b];
  const int nlist = idx ? K : (int)min<int64_t>(window, ri.p + 1);
  const int64_t jw0 = ri.p - nlist + 1;  // window mode: first position
  const int hi = min(nlist, lo + rows_per_split);
  const uint32_t jmax = (uint32_t)min<int64_t>(ri.p, (int64_t)INT32_MAX);
  if (idx) {
#pragma unroll
    for (int r = 0; r < PT; ++r)
      idx_lds[threadIdx.x + 256 * r] = (uint32_t)iv[r] <= jmax ? iv[r] : -1;
    if ((int)threadIdx.x < kIdxPad) idx_lds[kAttnMaxRows + threadIdx.x] = -1;
  }

  // q as the B operand of S^T: column = head 32 hb + l % 32, k = dims 16 s + 8 g + 0..7.
  // Heads past Hq repeat the last head; their results are never written.
  bf16x8 qb[KS];
  {
    const int hc = min(32 * hb + (l & 31), Hq - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qb[s] = as_bf16x8(ld16(q + ((int64_t)t * Hq + hc) * D + 16 * s + 8 * g));
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};

  // The workgroup works in steps of STEP index rows; row block rb (32 rows)
  // of a step is shared by the HB head-block waves rb * HB .. rb * HB + HB - 1,
  // and each of its K and V rows is fetched once per workgroup: with two
  // head blocks, wave hb = 0 loads the K rows and wave hb = 1 the V rows.
  // A step's rows are loaded into registers during the previous step (in
  // the gather layout of RowTile); at the step's start they go to LDS
  // (double-buffered tiles, one barrier per step) and every wave reads its
  // K operands and V transposes from there.  The row indices come from LDS,
  // so the only memory loads in flight are the row prefetches.
  constexpr int KB = VT::kLoads;  // 16-byte chunks per lane and tile
  static_assert(KB * 64 * 16 == VT::kBytes, "tile gather");
  auto tile = [&](int b, int r, int kind) {
    return smem + ((b * RB + r) * 2 + kind) * VT::kBytes;
  };
  const int G = l >> 4, jj = l & 15;
  // K/V row of list entry lp (lo <= lp < lo + rows_per_split + 2 STEP) in
  // index mode (IM) or window mode; invalid entries (past the list, or
  // outside [0, p]) map to row 0 of the sequence, so no gather leaves the
  // sequence's rows.  Index mode reads the staged, already checked entry
  // (-1 if invalid); window mode tests its position with one unsigned
  // compare (0 <= j <= p).
  auto row_of = [&](auto im, int lp, bool* ok) {
    if constexpr (decltype(im)::value) {
      const int32_t j = idx_lds[lp - lo];
      *ok = j >= 0;
      return max(j, 0);
    } else {
      const int32_t j = (int32_t)jw0 + lp;
      const bool v = (lp < hi) & ((uint32_t)j <= jmax);
      *ok = v;
      return v ? j : 0;
    }
  };
  // gather layout: this lane's chunk and its tile rows (one per load); row
  // j of the sequence is at 32-bit element offset j * D from these bases
  const int gch = l % VT::kNC, grow = l / VT::kNC;
  const uint16_t* const kbase = kc + row0 * D + 8 * gch;
  const uint16_t* const vbase = vc + row0 * D + 8 * gch;
  // steps of the workgroup (uniform: every wave passes every barrier; rows
  // past hi are masked)
  const int nsteps = hi > lo ? (hi - lo + STEP - 1) / STEP : 0;
  lds_barrier();  // the index rows are in LDS
  // The step loop, compiled once per wave role (LK: loads the K rows, LV:
  // loads the V rows), so each role holds only its own prefetch registers.
  auto run = [&](auto lk, auto lv, auto im) {
    constexpr bool LK = decltype(lk)::value, LV = decltype(lv)::value;
    u32x4 pk[KB], pv[KB];  // this lane's chunks of the next step's rows
    // rows of step i's tile of row block rb (invalid ones read row 0 of
    // the sequence; they are masked)
    auto load_rows = [&](int i, const uint16_t* base, u32x4 (&p)[KB]) {
      uint32_t rows[KB];  // every index read before any load is issued
#pragma unroll
      for (int c = 0; c < KB; ++c) {
        bool ok;
        rows[c] = (uint32_t)row_of(im, lo + STEP * i + 32 * rb + VT::kRPI * c + grow, &ok);
      }
#pragma unroll
      for (int c = 0; c < KB; ++c) p[c] = ld16(base + rows[c] * (uint32_t)D);
    };
    auto store_rows = [&](uint8_t* t, const u32x4 (&p)[KB]) {
#pragma unroll
      for (int c = 0; c < KB; ++c)
        *reinterpret_cast<u32x4*>(t + VT::offset(VT::kRPI * c + grow, 8 * gch)) = p[c];
    };
    bool valid;
    row_of(im, lp0, &valid);
    if (nsteps > 0) {
      if constexpr (LK) load_rows(0, kbase, pk);
      if constexpr (LV) load_rows(0, vbase, pv);
    }
#pragma unroll 1
    for (int i = 0; i < nsteps; ++i) {
      const int buf = i & 1;
      // this step's rows to LDS
      if constexpr (LK) store_rows(tile(buf, rb, 0), pk);
      if constexpr (LV) store_rows(tile(buf, rb, 1), pv);
      dma_barrier();  // the step's tiles are complete; the other buffer is free
      if (i + 1 < nsteps) {
        if constexpr (LK) load_rows(i + 1, kbase, pk);
        if constexpr (LV) load_rows(i + 1, vbase, pv);
      }
      bool valid_n = false;
      row_of(im, lp0 + STEP * (i + 1), &valid_n);
      const uint32_t vmask = (uint32_t)__ballot(valid);
      // S^T = K . q^T: the A operand of k-step s is row l % 32, dims
      // 16 s + 8 g .. + 7
      f32x16 sacc = {};
      {
        const uint8_t* kt = tile(buf, rb, 0);
        u32x4 kf[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
          kf[s] = *reinterpret_cast<const u32x4*>(kt + VT::offset(l & 31, 16 * s + 8 * g));
#pragma unroll
        for (int s = 0; s < KS; ++s) sacc = mfma32(as_bf16x8(kf[s]), qb[s], sacc);
      }
      // online softmax per head (exp2 domain).  The running max m_run moves
      // only when some head's step max passes it by more than kRescale (a
      // wave-uniform decision), so most steps leave O unscaled; the weights
      // exp2(c s - m_run) then stay below 2^kRescale, and the result, O / l,
      // does not depend on the reference point.  c > 0, so the max of the
      // raw logits gives the max of the scaled ones.
      float mx = -INFINITY;
      if (vmask == 0xffffffffu) {  // every row of the step valid
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ir = 8 * (r >> 2) + 4 * g + (r & 3);
          if (!((vmask >> ir) & 1u)) sacc[r] = -INFINITY;
          mx = fmaxf(mx, sacc[r]);
        }
      }
      mx = xor32_max(mx) * scale_log2;
      const bool grow = __ballot(mx > m_run + kRescale) != 0;
      float alpha = 1.f;
      if (grow) {
        const float m_new = fmaxf(m_run, mx);
        alpha = (m_new == -INFINITY) ? 1.f : fexp2(m_run - m_new);
        m_run = m_new;
      }
      // a head with no valid key yet keeps m_run = -inf; its weights are 0
      const float mu = (m_run == -INFINITY) ? 0.f : m_run;
      float sv[16];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[r] = fexp2(fmaf(sacc[r], scale_log2, -mu));
        psum += sv[r];
      }
      l_run = l_run * alpha + xor32_add(psum);
      bf16x8 pb[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[s2][e] = static_cast<__bf16>(sv[8 * s2 + e]);
      // O^T += V^T . P^T.  k slot e of step s2 is accumulator row
      // 16 s2 + 8 (e / 4) + 4 g + e % 4, so the A operand's 8 rows for half g
      // are two 4-row groups; each comes from one transpose read: lane jj of
      // a 16-lane group addresses row k0 + jj / 4, dims n0 + 4 (jj % 4) .. + 3.
      const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(tile(buf, rb, 1));
      u32x2 av[DB][2][2];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int n0 = 32 * db + 16 * (G & 1) + 4 * (jj & 3);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int k0 = 16 * s2 + 4 * g + (jj >> 2);
          av[db][s2][0] = lds_read_tr16(vt16 + VT::offset(k0, n0) / 2);
          av[db][s2][1] = lds_read_tr16(vt16 + VT::offset(k0 + 8, n0) / 2);
        }
      }
      if (grow) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          o[db] = mfma32(as_bf16x8(u32x4{av[db][s2][0][0], av[db][s2][0][1], av[db][s2][1][0],
                                         av[db][s2][1][1]}),
                         pb[s2], o[db]);
      }
      valid = valid_n;
    }
  };
  using T1 = std::integral_constant<bool, true>;
  using T0 = std::integral_constant<bool, false>;
  auto run_mode = [&](auto lk, auto lv) {
    if (idx)
      run(lk, lv, T1{});
    else
      run(lk, lv, T0{});
  };
  if constexpr (HB == 1)
    run_mode(T1{}, T1{});
  else if (hb == 0)
    run_mode(T1{}, T0{});
  else
    run_mode(T0{}, T1{});

  // ---- merge the RB row-block waves of each head block pairwise through LDS ----
  float* ms = reinterpret_cast<float*>(smem);
  auto put = [&](int slot) {
    float* dst = ms + (slot * HB + hb) * 64 * ST_FLOATS;
    dst[l] = m_run;
    dst[64 + l] = l_run;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(2 + db * 16 + r) * 64 + l] = o[db][r];
  };
  auto take = [&](int slot) {
    const float* src = ms + (slot * HB + hb) * 64 * ST_FLOATS;
    const float mo = src[l], lo2 = src[64 + l];
    const float M = fmaxf(m_run, mo);
    const float a = (M == -INFINITY) ? 0.f : fexp2(m_run - M);
    const float bb = (M == -INFINITY) ? 0.f : fexp2(mo - M);
    l_run = l_run * a + lo2 * bb;
    m_run = M;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a + src[(2 + db * 16 + r) * 64 + l] * bb;
  };
  lds_barrier();  // every wave is done with its V tile
  if constexpr (RB == 4) {
    if (rb >= 2) put(rb - 2);
    lds_barrier();
    if (rb < 2) take(rb);
    lds_barrier();
  }
  if (rb == 1) put(0);
  lds_barrier();
  if (rb != 0) return;
  take(0);

  // ---- the row-block-0 wave of each head block writes the result ----
  const int head = 32 * hb + (l & 31);
  if (head >= Hq) return;
  constexpr bool final_out = FINAL;  // one split: gated bf16 output, else partials
  const float Lsum = l_run, M = m_run;
  const float inv = (Lsum > 0.f) ? frcp(Lsum) : 0.f;
  float* pp = part + (((int64_t)t * nsplit + split) * Hq + head) * (D + 2);
  // gate values of this lane's outputs, all loaded before any is used
  // (gstride == 0: one gate value per head, broadcast over the head's dims)
  u32x2 gw[DB][4];
  float gsc = 1.f;
  if (final_out && gate) {
    if (gstride) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          gw[db][r4] = *reinterpret_cast<const u32x2*>(gate + ((int64_t)t * Hq + head) * D +
                                                       32 * db + 8 * r4 + 4 * g);
    } else {
      gsc = sigmoidf(bf16_to_f32(gate[(int64_t)t * Hq + head]));
    }
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * db + 8 * r4 + 4 * g;
      if constexpr (final_out) {
        uint16_t ob[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = o[db][4 * r4 + e] * inv;
          if (gate) {
            if (gstride) {
              const uint32_t wd = gw[db][r4][e >> 1];
              v *= sigmoidf(bf16_to_f32((uint16_t)((e & 1) ? (wd >> 16) : (wd & 0xffffu))));
            } else {
              v *= gsc;
            }
          }
          ob[e] = f32_to_bf16(v);
        }
        uint16_t* op = out + ((int64_t)t * Hq + head) * D + d0;
        *reinterpret_cast<u32x2*>(op) = u32x2{(uint32_t)ob[0] | ((uint32_t)ob[1] << 16),
                                             (uint32_t)ob[2] | ((uint32_t)ob[3] << 16)};
      } else {
        *reinterpret_cast<f32x4*>(pp + d0) =
            f32x4{o[db][4 * r4], o[db][4 * r4 + 1], o[db][4 * r4 + 2], o[db][4 * r4 + 3]};
      }
    }
  }
  if (g == 0) {
    if (final_out) {
      if (lse) lse[(int64_t)t * Hq + head] = (Lsum > 0.f) ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
    } else {
      pp[D] = M;
      pp[D + 1] = Lsum;
    }
  }
}

// Merge split partials: grid (T, Hq), one wave; lane i owns dims
// i*D/64 .. +D/64-1.  Every load is issued up front (one round trip): each
// lane reads its dims of every split's O (NS >= nsplit loads, indices past
// nsplit repeat the last split and get weight 0) and the (m, l) of split i;
// the (m, l) go through LDS.
constexpr int kMaxSplit = 64;

template <int D, int NS>
__global__ __launch_bounds__(64) void attn_combine_kernel(const float* __restrict__ part, int nsplit,
                                                          int Hq, const uint16_t* __restrict__ gate,
                                                          int gstride, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  constexpr int PL = D / 64;  // dims per lane (1 or 2)
  static_assert(NS <= 64 && (PL == 1 || PL == 2), "combine shape");
  __shared__ float sm_m[NS], sm_l[NS];
  const int t = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  const float* pp = part + ((int64_t)t * nsplit * Hq + h) * (D + 2);
  const int64_t stride = (int64_t)Hq * (D + 2);
  const int64_t off = ((int64_t)t * Hq + h) * D + PL * i;
  float ov[NS][PL];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float* src = pp + min(s, nsplit - 1) * stride + PL * i;
    if constexpr (PL == 2) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(src);
      ov[s][0] = v[0];
      ov[s][1] = v[1];
    } else {
      ov[s][0] = *src;
    }
  }
  const int si = min(i, nsplit - 1);
  const f32x2 ml = *reinterpret_cast<const f32x2*>(pp + si * stride + D);
  uint32_t graw = 0;
  if (gate) {
    if (!gstride) {  // one gate value per head
      graw = gate[(int64_t)t * Hq + h];
      graw |= graw << 16;
    } else if constexpr (PL == 2) {
      graw = *reinterpret_cast<const uint32_t*>(gate + off);
    } else {
      graw = gate[off];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (i < NS) {
    sm_m[i] = i < nsplit ? ml[0] : -INFINITY;
    sm_l[i] = ml[1];
  }
  lds_barrier();
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) M = fmaxf(M, sm_m[s]);
  float L = 0.f, acc[PL] = {};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float wgt = (s < nsplit && M != -INFINITY) ? fexp2(sm_m[s] - M) : 0.f;
    L += wgt * sm_l[s];
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] += wgt * ov[s][e];
  }
  const float inv = L > 0.f ? frcp(L) : 0.f;
  uint16_t ob[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) {
    float v = acc[e] * inv;
    if (gate) v *= sigmoidf(bf16_to_f32((uint16_t)(graw >> (16 * e))));
    ob[e] = f32_to_bf16(v);
  }
  if constexpr (PL == 2) *reinterpret_cast<uint32_t*>(out + off) = (uint32_t)ob[0] | ((uint32_t)ob[1] << 16);
  else out[off] = ob[0];
  if (lse && i == 0) lse[(int64_t)t * Hq + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int D>
static void launch_combine(int T, int Hq, const float* part, int nsplit, const uint16_t* gate,
                           int gstride, uint16_t* out, float* lse, hipStream_t stream) {
  const dim3 grid(T, Hq);
  if (nsplit <= 8)
    hipLaunchKernelGGL((attn_combine_kernel<D, 8>), grid, dim3(64), 0, stream, part, nsplit, Hq,
                       gate, gstride, out, lse);
  else if (nsplit <= 16)
    hipLaunchKernelGGL((attn_combine_kernel<D, 16>), grid, dim3(64), 0, stream, part, nsplit, Hq,
                       gate, gstride, out, lse);
  else if (nsplit <= 32)
    hipLaunchKernelGGL((attn_combine_kernel<D, 32>), grid, dim3(64), 0, stream, part, nsplit, Hq,
                       gate, gstride, out, lse);
  else
    hipLaunchKernelGGL((attn_combine_kernel<D, 64>), grid, dim3(64), 0, stream, part, nsplit, Hq,
                       gate, gstride, out, lse);
}

hipError_t launch_attn_combine(int T, int Hq, int D, const float* part, int nsplit,
                               const void* gate, int gstride, void* out, float* lse,
                               hipStream_t stream) {
  auto gp = static_cast<const uint16_t*>(gate);
  auto op = static_cast<uint16_t*>(out);
  if (D == 128 && Hq == 64)
    launch_combine<128>(T, Hq, part, nsplit, gp, gstride, op, lse, stream);
  else if (D == 64 && Hq == 8)
    launch_combine<64>(T, Hq, part, nsplit, gp, gstride, op, lse, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

AttnPlan attn_plan(int T, int K, int window, int Hq, int D) {
  AttnPlan p;
  const int nlist = K > 0 ? K : window;
  const int hb = (Hq + 31) / 32;
  const int step = 32 * (4 / (hb > 2 ? 2 : hb));  // rows per workgroup step
  // a step per workgroup when few queries, otherwise whole rows
  int rows = step;
  if ((int64_t)T * ((nlist + step - 1) / step) > 2048) rows = nlist > 0 ? nlist : step;
  while ((nlist + rows - 1) / rows > kMaxSplit) rows *= 2;
  if (K > 0 && rows > kAttnMaxRows) rows = kAttnMaxRows;  // the index rows fit the LDS
  p.rows_per_split = rows;
  p.nsplit = (nlist + rows - 1) / rows;
  if (p.nsplit < 1) p.nsplit = 1;
  p.ws_bytes = p.nsplit > 1 ? (size_t)T * p.nsplit * Hq * (D + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* idx, int K, int window, const void* gate,
                              int gstride, float sm_scale, int Hq, int D, const int32_t* cu_q,
                              const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                              void* out, float* lse, void* ws, const AttnPlan& plan,
                              hipStream_t stream, const AttnLayers* layers) {
  const float scale = (sm_scale != 0.f ? sm_scale : 1.f / sqrtf((float)D)) * kLog2e;
  auto qp = static_cast<const uint16_t*>(q);
  auto kp = static_cast<const uint16_t*>(k_cache);
  auto vp = static_cast<const uint16_t*>(v_cache);
  auto gp = static_cast<const uint16_t*>(gate);
  auto op = static_cast<uint16_t*>(out);
  float* part = static_cast<float*>(ws);
  AttnLayers one;
  one.n = 0;
  const AttnLayers& lay = layers ? *layers : one;
  dim3 grid(plan.nsplit, T, lay.n > 0 ? lay.n : 1);
  const bool final_out = plan.nsplit == 1;
  if (lay.n > 0 && !final_out) return hipErrorInvalidValue;  // layers: unsplit plans only
#define DSA_ATTN_LAUNCH(D_, HB_)                                                               \
  if (final_out)                                                                               \
    hipLaunchKernelGGL((sparse_attn_kernel<D_, HB_, true>), grid, dim3(256), 0, stream, qp, kp, \
                       vp, idx, K, window, gp, gstride, scale, Hq, cu_q, ctx_len, cu_ctx, B,   \
                       plan.rows_per_split, op, lse, part, plan.nsplit, lay);                  \
  else                                                                                         \
    hipLaunchKernelGGL((sparse_attn_kernel<D_, HB_, false>), grid, dim3(256), 0, stream, qp,   \
                       kp, vp, idx, K, window, gp, gstride, scale, Hq, cu_q, ctx_len, cu_ctx, B,\
                       plan.rows_per_split, op, lse, part, plan.nsplit, lay);
  if (D == 128 && Hq == 64) {
    DSA_ATTN_LAUNCH(128, 2)
    if (!final_out) launch_combine<128>(T, Hq, part, plan.nsplit, gp, gstride, op, lse, stream);
  } else if (D == 64 && Hq == 8) {
    DSA_ATTN_LAUNCH(64, 1)
    if (!final_out) launch_combine<64>(T, Hq, part, plan.nsplit, gp, gstride, op, lse, stream);
  } else {
    return hipErrorInvalidValue;
  }
#undef DSA_ATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace dsa
