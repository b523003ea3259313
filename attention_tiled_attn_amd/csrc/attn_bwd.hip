// attn_bwd.hip - attention backward for gfx950 (MI355X, CDNA4), bf16.
//
// Gradients of L = sum(O * dO) for the forward of attn_fwd_pp.hip. The pages
// name the backward pass and a deterministic mode for it without formulas
// (Neuron FA4 explainer, "FlashAttention-4: Built for Blackwell", backward-pass
// fixes); differentiating the definition gives, per query row q, with
// P = exp(s' - LSE) recomputed from the forward's LSE:
//
//     dV += P^T dO,  dP = dO V^T,  dS' = P * (dP - delta),  delta = rowsum(dO * O)
//     dS  = dS' * ds'/ds  (1, or 1 - tanh^2 for soft-capping)
//     dQ  = scale * dS K,  dK += scale * dS^T Q
//
// Two kernels per call, no atomics (every gradient element is summed by one
// lane in a fixed order, so results are reproducible bit for bit):
//  * attn_bwd_dq_kernel: one workgroup (4 waves x 32 rows) per 128 query rows
//    of one (batch, head); it first forms delta for its rows (written to the
//    caller's scratch for the second kernel), then walks the key tiles its
//    half of the block mask admits, in 32-key stages: S^T = K Q^T and
//    dP^T = V dO^T (A operands K and V rows), then dQ^T += K^T dS^T (A operand
//    K^T through transposing LDS reads). Two of these workgroups share a CU
//    at D <= 128.
//  * attn_bwd_dkdv2_kernel (D = 64, 128): one workgroup of eight waves per
//    128 keys of one (batch, key/value head), in pairs that own 32 keys: the
//    first wave of a pair forms S = Q K^T, P and dV^T += dO^T P and hands P
//    to its partner through LDS; the partner forms dP = dO V^T and, one stage
//    later, dS and dK^T += Q^T dS. Each wave holds one operand set and one
//    accumulator, so two waves share each SIMD.
//  * attn_bwd_dkdv_kernel (D = 256): one workgroup (4 waves x 32 keys) per
//    128 keys, each wave holding K^T, V^T and both accumulators: S = Q K^T
//    and dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS, one wave per SIMD.
// Both dK/dV kernels walk the query heads of the group and the query stages
// (64 rows, 32 at D = 256) that can see their keys.
// Tiles go from HBM/L2 straight into LDS (buffer-to-LDS copies into rings of
// stage buffers), rows unpadded with 16-byte chunks permuted so that both the
// b128 row reads and the transposing reads are free of bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_util.h"
#include "launch.h"
#include "variants.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kThreads = 256;   // 4 waves
constexpr int kRows = 128;      // query rows (dq) or keys (dkdv) per workgroup
constexpr int kTile = 128;      // key tile of the block mask
constexpr int kXcds = 8;

template <int D, int STAGE>
struct BGeo {
  // keys (dq) or query rows (dkdv) per stage
  static constexpr int kStage = STAGE;
  static constexpr int kKB = kStage / 32;              // 32-row blocks of a stage
  static constexpr int kCH = kStage / 16;              // 16-row chunks of a stage
  static constexpr int kSPT = kTile / kStage;          // stages per 128-key tile
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBufBytes = kStage * D * 2;     // one stage tile
  static constexpr int kCpr = D / 8;                   // 16-byte chunks per row
  static constexpr int kDma = kBufBytes / 1024 / 4;    // 1 KB copies per wave and tile
  static_assert(kDma >= 1 && kBufBytes % 4096 == 0, "stage geometry");
};

// Chunk permutation of a row-major tile read both ways: the 16 rows a
// quarter-wave reads in one b128 row-fragment read hit 16 different chunk
// positions, and the 4 consecutive rows a half-wave reads in one transposing
// read hit 4 different aligned groups of 4 chunks.
// (Banks repeat every 16 chunks, so D = 256 rows take D = 128's permutation
// of the low four chunk bits.)
template <int D>
__device__ inline int swz(int r) {
  if constexpr (D >= 128) return 4 * (r & 3) + ((r >> 2) & 3);
  const int pr = r >> 1;
  return 4 * (pr & 1) + ((pr >> 1) & 3);
}

template <int D>
__device__ inline unsigned row_off(int r, int chunk) {
  return static_cast<unsigned>(r * (D * 2) + ((chunk ^ swz<D>(r)) * 16));
}

// Copy one stage of rows of D bf16 starting at byte `gbase` of the slice behind `desc`
// (rows `grb` bytes apart) into a stage buffer, shared by WAVES waves: this
// wave fills 1 KB runs wq * n + j (n = runs per wave); lane i writes slot i,
// i.e. row s / kCpr at chunk position s % kCpr.
template <int D, int STAGE, int WAVES = 4>
__device__ inline void copy_tile(u32x4 desc, unsigned gbase, unsigned grb, unsigned lds_base, int wq, int lane) {
  using G = BGeo<D, STAGE>;
  constexpr int n = G::kBufBytes / 1024 / WAVES;
  static_assert(n >= 1 && n * 1024 * WAVES == G::kBufBytes, "copy shares");
#pragma unroll
  for (int j = 0; j < n; ++j) {
    const int s = (wq * n + j) * 64 + lane;
    const int r = s / G::kCpr, pos = s % G::kCpr;
    const unsigned goff = static_cast<unsigned>(r) * grb + static_cast<unsigned>((pos ^ swz<D>(r)) * 16);
    copy_to_lds(desc, gbase + goff, __builtin_amdgcn_readfirstlane(lds_base + (wq * n + j) * 1024));
  }
}

// A fragment of X^T for a 32x32x16 MFMA, from a row-major stage tile X (rows =
// the reduction index): lane (d = 32 db + l32, half g) gets rows
// 16 ch + 8 j + 4 g + 0..3 for j = 0, 1 at column d, through two transposing
// reads. toff[db][j] is this lane's offset for ch = 0.
template <int D>
__device__ inline bf16x8 trans_frag(const unsigned char* buf, unsigned toff0, unsigned toff1, int ch) {
  const unsigned char* a0 = buf + toff0 + 16 * ch * (D * 2);
  const unsigned char* a1 = buf + toff1 + 16 * ch * (D * 2);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
  const i16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

// Per-lane offsets of trans_frag for ch = 0: 16-lane group G16, lane sl reads
// 4 columns of row 8 j + 4 (G16 / 2) + sl / 4 starting at
// d = 32 db + 16 (G16 % 2) + 4 (sl % 4).
template <int D>
__device__ inline unsigned trans_off(int lane, int db, int j) {
  const int G16 = lane >> 4, sl = lane & 15;
  const int r = 8 * j + 4 * (G16 >> 1) + (sl >> 2);
  const int d0 = 32 * db + 16 * (G16 & 1) + 4 * (sl & 3);
  return row_off<D>(r, d0 >> 3) + (d0 & 7) * 2;
}

// Scheduling pattern for a run of N matrix-product groups whose LDS operand
// reads are independent of earlier products: the reads of the first AHEAD
// groups, then each group's products followed by the reads of the group
// AHEAD later. A group is one product per chain (G = products per group:
// reads per group = READS); used right after the code it orders.
// (AHEAD is clamped below N.)
template <int N, int AHEAD, int READS, int G = (READS == 3 ? 2 : 1)>
__device__ inline void reads_ahead() {
  constexpr int A = AHEAD < N ? AHEAD : N - 1;
  static_assert(A >= 1, "pipeline depth");
  __builtin_amdgcn_sched_group_barrier(0x100, A * READS, 0);
#pragma unroll
  for (int i = 0; i < N - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, G, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
  }
#pragma unroll
  for (int i = 0; i < A; ++i) __builtin_amdgcn_sched_group_barrier(0x008, G, 0);
}

// Modified score in log2 units, and d s'/d s for the chain rule.
template <int MOD>
__device__ inline float mod_score(float s, const VariantArgs& va, float slope2, lds_cf32* tab, int dk,
                                 float& dmod) {
  if constexpr (MOD == kModRelBias) {
    dmod = 1.f;
    const int d = min(max(dk, -va.rel_max), va.rel_max);
    return __builtin_fmaf(tab[d], kLog2e, s * va.c1);
  } else if constexpr (MOD == kModAlibi) {
    dmod = 1.f;
    return __builtin_fmaf(s, va.c1, slope2 * static_cast<float>(dk));
  } else if constexpr (MOD == kModSoftcap) {
    const float e = __builtin_amdgcn_exp2f(s * va.sc_in);
    const float th = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
    dmod = __builtin_fmaf(-th, th, 1.0f);
    return th * va.sc_out;
  } else {
    dmod = 1.f;
    return s * va.c1;
  }
}

// ---------------------------------------------------------------------------
// Stage sizes. dQ: 32 keys per stage at every D, which keeps a workgroup
// under 64 KB of LDS and a wave under 256 registers at D <= 128, so two
// workgroups share a CU (two waves per SIMD: one's matrix products overlap
// the other's vector work). dK/dV: 64 query rows (32 at D = 256, where a
// 64-row tile would not leave room for the three-stage rings); at D = 64 and
// 128 two waves split each key block's work and share a SIMD, at D = 256 one
// wave per SIMD holds the accumulators and K^T, V^T fragments (more than 256
// registers).
template <int D> constexpr int kDqStage = 32;
template <int D> constexpr int kDkvStage = D == 256 ? 32 : 64;
// waves per SIMD; at D = 64 three dQ workgroups share a CU (registers under
// 168 and 41-45 KB of LDS each): alibi_d64 backward +2.7%, doc_swa at D = 64
// +6% against two (A/B on one machine)
template <int D> constexpr int kDqWaves = D == 256 ? 1 : D == 64 ? 3 : 2;

// dQ (and delta)
template <int D, int MOD, bool DOCS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kDqWaves<D>, kDqWaves<D>)))
void attn_bwd_dq_kernel(BwdLaunch p, const int* __restrict__ kv_count, const int* __restrict__ kv_list) {
  using G = BGeo<D, kDqStage<D>>;
  constexpr int DC = D / 16, DB = D / 32, RB = G::kRowBytes;
  constexpr int kStage = G::kStage, KB = G::kKB, CH = G::kCH, SPT = G::kSPT;
  // a ring of four stages: stage t is read for S^T, dP^T in iteration t and
  // for the dQ products in iteration t + 1, while stage t + 2 arrives
  constexpr int kRing4 = 4;
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[kRing4 * G::kBufBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[kRing4 * G::kBufBytes];
  // list entries (kv_tile << 4) | class bits, kv_tile < kPairMaxKeyTiles;
  // with the relative-bias table they are stored in 16 bits, so that two
  // workgroups still fit one CU's LDS at D = 128
  using Ent = std::conditional_t<MOD == kModRelBias, unsigned short, int>;
  static_assert(kPairMaxKeyTiles << 4 <= 65536, "16-bit list entries");
  __shared__ Ent ents[kPairMaxKeyTiles];
  __shared__ int n_ent_lds;
  __shared__ float rtab[MOD == kModRelBias ? kRelCap : 1];   // this head's bias table

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const int nq = (p.Sq + kRows - 1) / kRows;
  const int total = p.B * p.H * nq;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int lin = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (lin >= total) return;
  const int qt = nq - 1 - (lin % nq);
  const int bh = lin / nq;
  const int h = bh % p.H, b = bh / p.H;
  const int kvh = h / (p.H / p.Hkv);
  const size_t q_head = (static_cast<size_t>(b) * p.H + h) * p.Sq;   // LSE and delta rows
  // row strides in bytes; each slice's resource ends after its last row, so
  // rows past the end read as zero
  const unsigned qrb = static_cast<unsigned>(p.q_sr) * 2u, orb = static_cast<unsigned>(p.o_sr) * 2u;
  const unsigned krb = static_cast<unsigned>(p.k_sr) * 2u, vrb = static_cast<unsigned>(p.v_sr) * 2u;
  const rsrc_t rq = make_rsrc(static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh,
                              static_cast<unsigned>(p.Sq - 1) * qrb + RB);
  const rsrc_t ro = make_rsrc(static_cast<const __bf16*>(p.out) + b * p.o_sb + h * p.o_sh,
                              static_cast<unsigned>(p.Sq - 1) * orb + RB);
  const rsrc_t rdo = make_rsrc(static_cast<const __bf16*>(p.dout) + b * p.o_sb + h * p.o_sh,
                               static_cast<unsigned>(p.Sq - 1) * orb + RB);
  const u32x4 kdesc = make_desc(static_cast<const __bf16*>(p.k) + b * p.k_sb + kvh * p.k_sh,
                                static_cast<unsigned>(p.Skv - 1) * krb + RB);
  const u32x4 vdesc = make_desc(static_cast<const __bf16*>(p.v) + b * p.v_sb + kvh * p.v_sh,
                                static_cast<unsigned>(p.Skv - 1) * vrb + RB);

  const int q_row = qt * kRows + wave * 32 + l32;
  const bool q_ok = q_row < p.Sq;

  // key-tile list: half qt % 2 of 256-row tile qt / 2. Its length and its
  // first kThreads entries are fetched first (every list has room for nk
  // entries), so that they arrive with the rows below instead of after them.
  const int qp = qt >> 1, any_bit = 2 * (qt & 1), full_bit = any_bit + 1;
  const int bm_b = (kv_count && p.bm_num_b > 1) ? b : 0;
  const int* list = kv_count ? kv_list + (static_cast<size_t>(bm_b) * p.nq + qp) * p.nk : nullptr;
  const int n_listed = kv_count ? kv_count[bm_b * p.nq + qp] : p.nk;
  const int e_first = (list && tid < p.nk) ? list[tid] : 0;

  // B operands (Q^T, dO^T) and the O row for this row's delta = dO . O,
  // formed once the list is in place and the first key stages are on their
  // way (the rows arrive meanwhile)
  bf16x8 qf[DC], dof[DC], of[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const unsigned col = (c * 16 + g * 8) * 2;
    const unsigned qo = q_ok ? static_cast<unsigned>(q_row) * qrb + col : 0x80000000u;
    const unsigned oo = q_ok ? static_cast<unsigned>(q_row) * orb + col : 0x80000000u;
    qf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 0, 0));
    dof[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rdo, oo, 0, 0));
    of[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ro, oo, 0, 0));
  }
  const float lse_raw = q_ok ? p.lse[q_head + q_row] : -INFINITY;
  // exponent base in log2 units; a row that admitted nothing has P = 0
  const float lse2 = (lse_raw == -INFINITY) ? INFINITY : lse_raw * kLog2e;
  float slope2 = 0.f;
  if constexpr (MOD == kModAlibi) slope2 = p.va.slopes[h] * kLog2e;
  const int* doc_row = DOCS ? p.va.doc + static_cast<size_t>(b) * p.va.doc_stride : p.va.doc;
  const rsrc_t rdoc = make_rsrc(doc_row, DOCS ? static_cast<unsigned>(p.va.doc_stride) * 4u : 0u);
  const int q_pos = q_row + p.va.q_offset;   // position in the key sequence
  const int doc_q = (DOCS && q_ok) ? doc_row[q_pos] : 0;

  // The list names the key tiles that either half sees; wave 0 keeps, in
  // order, those this half sees (compacting in place: each 64-entry chunk is
  // read before any of it is written, and no entry moves up). Without a
  // block mask every key tile is visited as partial, except when there is no
  // mask at all: then a tile wholly inside Skv is full.
  auto unlisted = [&](int j) -> int {
    return (j << 4) | ((p.mask_kind == 0 && (j + 1) * kTile <= p.Skv) ? 0xF : 0);
  };
  if (tid < n_listed) ents[tid] = static_cast<Ent>(list ? e_first : unlisted(tid));
  for (int i = tid + kThreads; i < n_listed; i += kThreads) ents[i] = static_cast<Ent>(list ? list[i] : unlisted(i));
  if constexpr (MOD == kModRelBias) stage_rel_table(p.va, h, (lds_f32*)(rtab), tid, kThreads);
  lds_cf32* const tab = (lds_cf32*)(rtab) + p.va.rel_max;
  __syncthreads();
  if (list) {
    if (wave == 0) {
      int base = 0;
      for (int j0 = 0; j0 < n_listed; j0 += 64) {
        const int e = j0 + lane < n_listed ? ents[j0 + lane] : 0;
        const bool keep = j0 + lane < n_listed && ((e >> any_bit) & 1);
        const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
        const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(m), 0));
        if (keep) ents[base + rank] = static_cast<Ent>(e);
        base += __builtin_popcountll(m);
      }
      if (lane == 0) n_ent_lds = base;
    }
    __syncthreads();
  }
  const int n_entries = list ? __builtin_amdgcn_readfirstlane(n_ent_lds) : n_listed;
  int T = SPT * n_entries;
  if (n_entries > 0) {
    // stages of the last tile that start at or past Skv are dropped
    const int last = ents[n_entries - 1] >> 4;
    const int kept = (p.Skv - last * kTile + kStage - 1) / kStage;
    T -= SPT - min(kept, SPT);
  }
  auto ent = [&](int t) -> int { return ents[min(t, max(T - 1, 0)) / SPT]; };
  auto stage_kv0 = [](int t, int e) -> int { return (e >> 4) * kTile + (t % SPT) * kStage; };

  // fragment offsets formed as needed from one base each (the chunk
  // permutation XORs low bits only, so chunk c's row offset is chunk 0's
  // XOR 32 c and block db's transposed offset block 0's XOR 64 db)
  constexpr bool kXor = true;
  unsigned koff[kXor ? 1 : DC];
#pragma unroll
  for (int c = 0; c < (kXor ? 1 : DC); ++c) koff[c] = row_off<D>(l32, 2 * c + g);
  auto koff_at = [&](int c) -> unsigned { return kXor ? koff[0] ^ (c << 5) : koff[c]; };
  unsigned toff[kXor ? 1 : DB][2];
#pragma unroll
  for (int db = 0; db < (kXor ? 1 : DB); ++db)
#pragma unroll
    for (int j = 0; j < 2; ++j) toff[db][j] = trans_off<D>(lane, db, j);
  auto toff_at = [&](int db, int j) -> unsigned { return kXor ? toff[0][j] ^ (db << 6) : toff[db][j]; };

  const unsigned kl = lds_addr(kbuf), vl = lds_addr(vbuf);
  auto copy_stage = [&](int t, int ring) {
    const unsigned kv0 = static_cast<unsigned>(stage_kv0(t, __builtin_amdgcn_readfirstlane(ent(t))));
    copy_tile<D, kStage>(kdesc, kv0 * krb, krb, kl + ring * G::kBufBytes, wave, lane);
    copy_tile<D, kStage>(vdesc, kv0 * vrb, vrb, vl + ring * G::kBufBytes, wave, lane);
  };

  if (T > 0) copy_stage(0, 0);
  if (T > 1) copy_stage(1, 1);
  float delta = 0.f;
#pragma unroll
  for (int c = 0; c < DC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) delta = __builtin_fmaf(static_cast<float>(dof[c][e]), static_cast<float>(of[c][e]), delta);
  delta = sum_pair32(delta);
  if (q_ok && g == 0) p.delta[q_head + q_row] = delta;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  // dQ^T += K^T dS^T of one stage (slot `sl`), one iteration late, beside the
  // next stage's exponentials (as in the dK/dV kernel)
  bf16x8 dsf_prev[CH];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) dsf_prev[ch] = bf16x8{};
  auto dq_products = [&](int sl) {
    const unsigned char* kp_ = kbuf + sl * G::kBufBytes;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ch = 0; ch < CH; ++ch)
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(trans_frag<D>(kp_, toff_at(db, 0), toff_at(db, 1), ch),
                                                         dsf_prev[ch], dq[db], 0, 0, 0);
  };

  for (int t = 0; t < T; ++t) {
    const int ring = t % kRing4;
    const int e = __builtin_amdgcn_readfirstlane(ent(t));
    const bool full = ((e >> full_bit) & 1) != 0;
    const int kv0 = stage_kv0(t, e);
    const unsigned char* kb_ = kbuf + ring * G::kBufBytes;
    const unsigned char* vb_ = vbuf + ring * G::kBufBytes;

    // S^T = K Q^T, then dP^T = V dO^T, each in a scheduling region of its
    // own with its operand reads issued four products ahead (in one region
    // the compiler runs one chain ahead and fetches each of its operands
    // just before use). dP^T starts from zero and delta is subtracted after
    // the products: where P = 1 (a single admitted key) dP and delta are the
    // same dot product and then cancel exactly, as the definition's dS = 0.
    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = dp[kb] = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_ + koff_at(c) + kb * 32 * RB);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
      }
    reads_ahead<DC * KB, 4, 1>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(vb_ + koff_at(c) + kb * 32 * RB);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dof[c], dp[kb], 0, 0, 0);
      }
    reads_ahead<DC * KB, 4, 1>();
    __builtin_amdgcn_sched_barrier(0);

    // dS^T = P^T (dP^T - delta) ds'/ds, packed to bf16 in the key order of
    // the B operand (element 16 kb + r is key kv0 + 32 kb + 8 (r / 4) + 4 g + r % 4).
    // The modified scores are formed first and masked in place on partial
    // stages, so the exponentials share a block with the deferred products.
    float tt[KB * 16];
    float dmv[MOD == kModSoftcap ? KB * 16 : 1];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kidx = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        float dmod;
        // without a score mod the row's LSE joins the scale in one FMA (for a
        // row with no admitted key lse2 = +inf, so P = exp2(-inf) = 0)
        if constexpr (MOD == kModNone) tt[kb * 16 + r] = __builtin_fmaf(s[kb][r], p.va.c1, -lse2);
        else tt[kb * 16 + r] = mod_score<MOD>(s[kb][r], p.va, slope2, tab, kidx - q_pos, dmod);
        if constexpr (MOD == kModSoftcap) dmv[kb * 16 + r] = dmod;
      }
    if (!full) {
      // Element 16 kb + r is key kk0 + c with c = 32 kb + 8 (r / 4) + r % 4.
      // The key range, the causal part (with its prefix) and the window
      // admit c in [lo_c, hi_c]; a stage whose keys share one document label
      // folds the label test into that interval. Each test runs only when
      // some lane of the wave needs it (one compare and one select per element).
      const float ninf = -INFINITY;
      const int kk0 = kv0 + 4 * g;
      const long long d = static_cast<long long>(q_pos) - kk0;
      long long hi = static_cast<long long>(p.Skv) - 1 - kk0;
      if (p.mask_kind & kMaskCausal) hi = min(hi, max(d, static_cast<long long>(p.va.prefix) - 1 - kk0));
      const long long lo = (p.mask_kind & kMaskWindow) ? d - p.va.window + 1 : 0LL;
      int hi_c = static_cast<int>(min(max(hi, -1LL), static_cast<long long>(kStage)));
      const int lo_c = static_cast<int>(min(max(lo, 0LL), static_cast<long long>(kStage)));
      bool need_doc = false;
      if constexpr (DOCS) {
        const int lk = __builtin_amdgcn_raw_buffer_load_b32(
            rdoc, static_cast<unsigned>(kv0 + (lane & (kStage - 1))) * 4u, 0, 0);
        const int l0 = __builtin_amdgcn_readfirstlane(lk);
        if (__all(lk == l0)) {
          if (doc_q != l0) hi_c = -1;
        } else {
          need_doc = true;
        }
      }
      if (need_doc) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 l4 = __builtin_amdgcn_raw_buffer_load_b128(
                rdoc, static_cast<unsigned>(kk0 + 32 * kb + 8 * i) * 4u, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              mask_in_place(tt[kb * 16 + 4 * i + e],
                            __builtin_amdgcn_ballot_w64(static_cast<int>(l4[e]) == doc_q), ninf);
          }
      }
      if (!__all(lo_c <= 0)) {
#pragma unroll
        for (int j = 0; j < KB * 16; ++j)
          mask_in_place(tt[j], __builtin_amdgcn_ballot_w64((j >> 4) * 32 + 8 * ((j >> 2) & 3) + (j & 3) >= lo_c),
                        ninf);
      }
      if (!__all(hi_c >= kStage - 1)) {
#pragma unroll
        for (int j = 0; j < KB * 16; ++j)
          mask_in_place(tt[j], __builtin_amdgcn_ballot_w64((j >> 4) * 32 + 8 * ((j >> 2) & 3) + (j & 3) <= hi_c),
                        ninf);
      }
    }
    bf16x8 dsf[CH];
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      const int kb = ch >> 1, r0 = (ch & 1) * 8;
      unsigned w[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float v2[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int r = r0 + 2 * jj + x;
          const float pr = __builtin_amdgcn_exp2f(MOD == kModNone ? tt[kb * 16 + r] : tt[kb * 16 + r] - lse2);
          v2[x] = pr * (dp[kb][r] - delta);
          if constexpr (MOD == kModSoftcap) v2[x] *= dmv[kb * 16 + r];
        }
        w[jj] = pack_bf16(v2[0], v2[1]);
      }
      const u32x4 wv = {w[0], w[1], w[2], w[3]};
      dsf[ch] = __builtin_bit_cast(bf16x8, wv);
    }

    // the previous stage's dQ products (at t = 0 zero fragments on stage 0's
    // rows, which add exactly nothing)
    dq_products(t == 0 ? 0 : (t - 1) % kRing4);
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      asm volatile("" ::"v"(dsf[ch]));   // keeps dS in the products' block
      dsf_prev[ch] = dsf[ch];
    }

    // stage t + 2 into the slot stage t - 2 used; retire stage t + 1
    if (t + 2 < T) {
      copy_stage(t + 2, (t + 2) % kRing4);
      wait_vm<2 * G::kDma>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();
  }
  if (T > 0) dq_products((T - 1) % kRing4);

  if (q_ok) {
    __bf16* const drow = static_cast<__bf16*>(p.dq) + b * p.q_sb + h * p.q_sh + static_cast<size_t>(q_row) * p.q_sr;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        const u32x2 vv = {pack_bf16(dq[db][4 * i] * p.scale, dq[db][4 * i + 1] * p.scale),
                          pack_bf16(dq[db][4 * i + 2] * p.scale, dq[db][4 * i + 3] * p.scale)};
        *reinterpret_cast<u32x2*>(drow + d0) = vv;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV
template <int D, int MOD, bool DOCS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_dkdv_kernel(BwdLaunch p) {
  using G = BGeo<D, kDkvStage<D>>;
  constexpr int DC = D / 16, DB = D / 32, RB = G::kRowBytes;
  constexpr int kStage = G::kStage, KB = G::kKB, CH = G::kCH;
  // a ring of four stages: stage u is read for S, dP and P, dS in iteration
  // u, and again for dV, dK in iteration u + 1, while stage u + 2 arrives
  constexpr int kRing4 = 4;
  __shared__ __attribute__((aligned(1024))) unsigned char qbuf[kRing4 * G::kBufBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char obuf[kRing4 * G::kBufBytes];
  __shared__ __attribute__((aligned(16))) float lbuf[kRing4 * kDkvStage<D>];
  __shared__ __attribute__((aligned(16))) float dbuf[kRing4 * kDkvStage<D>];
  __shared__ float rtab[MOD == kModRelBias ? kRelCap : 1];   // the current head's bias table
  lds_cf32* const tab = (lds_cf32*)(rtab) + p.va.rel_max;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const int nk = (p.Skv + kRows - 1) / kRows;
  const int total = p.B * p.Hkv * nk;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int lin = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (lin >= total) return;
  const int kt = lin % nk;                  // ascending: under a causal mask the low tiles see the most rows
  const int bkh = lin / nk;
  const int kvh = bkh % p.Hkv, b = bkh / p.Hkv;
  const int rep = p.H / p.Hkv;
  // row strides in bytes; resources end after the slice's last row
  const unsigned qrb = static_cast<unsigned>(p.q_sr) * 2u, orb = static_cast<unsigned>(p.o_sr) * 2u;
  const unsigned krb = static_cast<unsigned>(p.k_sr) * 2u, vrb = static_cast<unsigned>(p.v_sr) * 2u;
  const rsrc_t rk = make_rsrc(static_cast<const __bf16*>(p.k) + b * p.k_sb + kvh * p.k_sh,
                              static_cast<unsigned>(p.Skv - 1) * krb + RB);
  const rsrc_t rv = make_rsrc(static_cast<const __bf16*>(p.v) + b * p.v_sb + kvh * p.v_sh,
                              static_cast<unsigned>(p.Skv - 1) * vrb + RB);

  const int k_row = kt * kRows + wave * 32 + l32;
  const bool k_ok = k_row < p.Skv;

  // B operands K^T and V^T: lane (key l32, half g) holds 8 consecutive d
  bf16x8 kf[DC], vf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const unsigned col = (c * 16 + g * 8) * 2;
    const unsigned ko = k_ok ? static_cast<unsigned>(k_row) * krb + col : 0x80000000u;
    const unsigned vo = k_ok ? static_cast<unsigned>(k_row) * vrb + col : 0x80000000u;
    kf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, ko, 0, 0));
    vf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, 0));
  }
  const int* doc_row = DOCS ? p.va.doc + static_cast<size_t>(b) * p.va.doc_stride : p.va.doc;
  const rsrc_t rdoc = make_rsrc(doc_row, DOCS ? static_cast<unsigned>(p.va.doc_stride) * 4u : 0u);
  const int doc_k = (DOCS && k_ok) ? doc_row[k_row] : 0;

  // the query stages that can see keys [k_lo, k_hi] of this tile
  // (query row r sits at position r + q_offset; keys below the prefix are
  // exempt from the causal part)
  const bool causal = p.mask_kind & kMaskCausal;
  const bool window = p.mask_kind & kMaskWindow;
  const int off = p.va.q_offset;
  const int k_lo = kt * kRows;
  const int k_hi = min(p.Skv, k_lo + kRows) - 1;
  const int q_first = (causal && k_lo >= p.va.prefix) ? min(max(k_lo - off, 0), p.Sq) : 0;
  const int q_end = window ? static_cast<int>(min(static_cast<long long>(p.Sq),
                                                  static_cast<long long>(k_hi) + p.va.window - off))
                           : p.Sq;
  const int s0 = q_first / kStage;
  const int ns = q_end > q_first ? (q_end + kStage - 1) / kStage - s0 : 0;
  const int T = rep * ns;

  // fragment offsets, formed as needed at D = 256 (as in the dQ kernel)
  constexpr bool kXor = D == 256;
  unsigned qoff[kXor ? 1 : DC];
#pragma unroll
  for (int c = 0; c < (kXor ? 1 : DC); ++c) qoff[c] = row_off<D>(l32, 2 * c + g);
  auto qoff_at = [&](int c) -> unsigned { return kXor ? qoff[0] ^ (c << 5) : qoff[c]; };
  unsigned toff[kXor ? 1 : DB][2];
#pragma unroll
  for (int db = 0; db < (kXor ? 1 : DB); ++db)
#pragma unroll
    for (int j = 0; j < 2; ++j) toff[db][j] = trans_off<D>(lane, db, j);
  auto toff_at = [&](int db, int j) -> unsigned { return kXor ? toff[0][j] ^ (db << 6) : toff[db][j]; };

  const unsigned ql = lds_addr(qbuf), ol = lds_addr(obuf);
  const unsigned ll = lds_addr(lbuf), dl = lds_addr(dbuf);
  // stage u: query head rep kvh + u / ns, rows kStage (s0 + u % ns) ..
  auto copy_stage = [&](int u, int ring) {
    const int hh = kvh * rep + u / ns;
    const int r0 = (s0 + u % ns) * kStage;
    const size_t q_head = (static_cast<size_t>(b) * p.H + hh) * p.Sq;   // LSE and delta rows
    const u32x4 qd = make_desc(static_cast<const __bf16*>(p.q) + b * p.q_sb + hh * p.q_sh,
                               static_cast<unsigned>(p.Sq - 1) * qrb + RB);
    const u32x4 od = make_desc(static_cast<const __bf16*>(p.dout) + b * p.o_sb + hh * p.o_sh,
                               static_cast<unsigned>(p.Sq - 1) * orb + RB);
    copy_tile<D, kStage>(qd, static_cast<unsigned>(r0) * qrb, qrb, ql + ring * G::kBufBytes, wave, lane);
    copy_tile<D, kStage>(od, static_cast<unsigned>(r0) * orb, orb, ol + ring * G::kBufBytes, wave, lane);
    if (wave == 0 && lane < kStage / 4) {
      // kStage floats of LSE and of delta, 16 bytes per lane
      const u32x4 lsd = make_desc(p.lse + q_head, static_cast<unsigned>(p.Sq) * 4u);
      const u32x4 dld = make_desc(p.delta + q_head, static_cast<unsigned>(p.Sq) * 4u);
      copy_to_lds(lsd, static_cast<unsigned>(r0) * 4u + lane * 16u,
                  __builtin_amdgcn_readfirstlane(ll + ring * kStage * 4));
      copy_to_lds(dld, static_cast<unsigned>(r0) * 4u + lane * 16u,
                  __builtin_amdgcn_readfirstlane(dl + ring * kStage * 4));
    }
  };
  auto retire = [&](bool issued) {
    // copies of the previous stage complete (wave 0 also copied LSE and delta)
    if (issued) {
      if (wave == 0) wait_vm<2 * G::kDma + 2>();
      else wait_vm<2 * G::kDma>();
    } else {
      wait_vm<0>();
    }
  };

  if (T > 0) copy_stage(0, 0);
  if (T > 1) copy_stage(1, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dkt[i] = dvt[i] = f32x16{};

  // dV^T += dO^T P and dK^T += Q^T dS of one stage (slot `sl`). They run one
  // iteration late, beside the next stage's vector work, which they do not
  // depend on: with one wave per SIMD this is where matrix and vector work
  // overlap.
  bf16x8 pf_prev[CH], dsf_prev[CH];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) pf_prev[ch] = dsf_prev[ch] = bf16x8{};
  auto dkdv_products = [&](int sl) {
    const unsigned char* qp_ = qbuf + sl * G::kBufBytes;
    const unsigned char* op_ = obuf + sl * G::kBufBytes;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(trans_frag<D>(op_, toff_at(db, 0), toff_at(db, 1), ch),
                                                          pf_prev[ch], dvt[db], 0, 0, 0);
        dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(trans_frag<D>(qp_, toff_at(db, 0), toff_at(db, 1), ch),
                                                          dsf_prev[ch], dkt[db], 0, 0, 0);
      }
  };

  for (int u = 0; u < T; ++u) {
    const int ring = u % kRing4;
    const int hh = kvh * rep + u / ns;
    const int r0 = (s0 + u % ns) * kStage;
    const unsigned char* qb_ = qbuf + ring * G::kBufBytes;
    const unsigned char* ob_ = obuf + ring * G::kBufBytes;
    const float* lb = lbuf + ring * kStage;
    const float* dlb = dbuf + ring * kStage;
    // every pair of the stage in range and admitted?
    const int q_last = r0 + kStage - 1;
    bool full = !DOCS && q_last < p.Sq && k_hi == k_lo + kRows - 1;
    if (causal) full = full && (r0 + off >= k_hi || k_hi < p.va.prefix);
    if (window) full = full && (q_last + off - k_lo < p.va.window);
    float slope2 = 0.f;
    if constexpr (MOD == kModAlibi) slope2 = p.va.slopes[hh] * kLog2e;
    if constexpr (MOD == kModRelBias) {
      // a new query head: its table replaces the last head's, whose last
      // reader finished before the previous stage's closing barrier
      if (u % ns == 0) {
        stage_rel_table(p.va, hh, (lds_f32*)(rtab), tid, kThreads);
        __syncthreads();
      }
    }

    // S = Q K^T and dP = dO V^T: KB 32-row query blocks
    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int qb = 0; qb < KB; ++qb) s[qb] = dp[qb] = f32x16{};
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int qb = 0; qb < KB; ++qb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(qb_ + qoff_at(c) + qb * 32 * RB);
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[c], s[qb], 0, 0, 0);
        const bf16x8 ao = *reinterpret_cast<const bf16x8*>(ob_ + qoff_at(c) + qb * 32 * RB);
        dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[c], dp[qb], 0, 0, 0);
      }

    // P and dS in the query order of the B operand (element 16 qb + i is row
    // r0 + 32 qb + 8 (i / 4) + 4 g + i % 4). The modified scores are formed
    // for every element first and masked in place on partial stages, so the
    // exponentials below sit in one block with the previous stage's
    // products, which the compiler can interleave with them.
    float tt[KB * 16];
    float dmv[MOD == kModSoftcap ? KB * 16 : 1];
#pragma unroll
    for (int qb = 0; qb < KB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qpos = r0 + 32 * qb + 8 * (i >> 2) + 4 * g + (i & 3) + off;
        float dmod;
        tt[qb * 16 + i] = mod_score<MOD>(s[qb][i], p.va, slope2, tab, k_row - qpos, dmod);
        if constexpr (MOD == kModSoftcap) dmv[qb * 16 + i] = dmod;
      }
    if (!full) {
      // Element 16 qb + i is query row rr0 + c with c = 32 qb + 8 (i / 4) +
      // i % 4, at position rr0 + c + off. The query range, the causal part
      // (keys below the prefix are seen by every row) and the window admit c
      // in [lo_c, hi_c] (none for a key past Skv); a stage whose rows share
      // one document label folds the label test into that interval. Each test
      // runs only when some lane of the wave needs it.
      const float ninf = -INFINITY;
      const int rr0 = r0 + 4 * g;
      const long long kq = static_cast<long long>(k_row) - off - rr0;   // the row at the key's position
      long long hi = static_cast<long long>(p.Sq) - 1 - rr0;
      if (window) hi = min(hi, kq + p.va.window - 1);
      if (!k_ok) hi = -1;
      const long long lo = (causal && k_row >= p.va.prefix) ? kq : 0LL;
      int hi_c = static_cast<int>(min(max(hi, -1LL), static_cast<long long>(kStage)));
      const int lo_c = static_cast<int>(min(max(lo, 0LL), static_cast<long long>(kStage)));
      bool need_doc = false;
      if constexpr (DOCS) {
        const int lq = __builtin_amdgcn_raw_buffer_load_b32(
            rdoc, static_cast<unsigned>(r0 + off + (lane & (kStage - 1))) * 4u, 0, 0);
        const int l0 = __builtin_amdgcn_readfirstlane(lq);
        if (__all(lq == l0)) {
          if (doc_k != l0) hi_c = -1;
        } else {
          need_doc = true;
        }
      }
      if (need_doc) {
#pragma unroll
        for (int qb = 0; qb < KB; ++qb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const u32x4 lab = __builtin_amdgcn_raw_buffer_load_b128(
                rdoc, static_cast<unsigned>(rr0 + 32 * qb + 8 * i4 + off) * 4u, 0, 0);
#pragma unroll
            for (int x = 0; x < 4; ++x)
              mask_in_place(tt[qb * 16 + 4 * i4 + x],
                            __builtin_amdgcn_ballot_w64(static_cast<int>(lab[x]) == doc_k), ninf);
          }
      }
      if (!__all(lo_c <= 0)) {
#pragma unroll
        for (int j = 0; j < KB * 16; ++j)
          mask_in_place(tt[j], __builtin_amdgcn_ballot_w64((j >> 4) * 32 + 8 * ((j >> 2) & 3) + (j & 3) >= lo_c),
                        ninf);
      }
      if (!__all(hi_c >= kStage - 1)) {
#pragma unroll
        for (int j = 0; j < KB * 16; ++j)
          mask_in_place(tt[j], __builtin_amdgcn_ballot_w64((j >> 4) * 32 + 8 * ((j >> 2) & 3) + (j & 3) <= hi_c),
                        ninf);
      }
    }
    bf16x8 pf[CH], dsf[CH];
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      const int qb = ch >> 1, i0 = (ch & 1) * 8;
      unsigned wp[4], wd[4];
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        // rows r0 + 32 qb + 8 (i / 4) + 4 g + 0..3 for i = i0 + 4 hv ..
        const int ql0 = 32 * qb + 8 * ((i0 >> 2) + hv) + 4 * g;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lb + ql0);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlb + ql0);
        float pv[4], dv4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = i0 + 4 * hv + x;
          // exp2(t - log2(e) LSE) as one FMA. A row with no admitted key
          // has LSE = -inf and every score masked to -inf; its LSE is
          // clamped (one med3) to -1e30 so that the FMA gives -inf (P = 0),
          // not NaN.
          const float lc = __builtin_amdgcn_fmed3f(l4[x], -1e30f, 3e38f);
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(lc, -kLog2e, tt[qb * 16 + i]));
          pv[x] = pr;
          dv4[x] = pr * (dp[qb][i] - d4[x]);
          if constexpr (MOD == kModSoftcap) dv4[x] *= dmv[qb * 16 + i];
        }
        wp[2 * hv] = pack_bf16(pv[0], pv[1]);
        wp[2 * hv + 1] = pack_bf16(pv[2], pv[3]);
        wd[2 * hv] = pack_bf16(dv4[0], dv4[1]);
        wd[2 * hv + 1] = pack_bf16(dv4[2], dv4[3]);
      }
      const u32x4 wpv = {wp[0], wp[1], wp[2], wp[3]};
      const u32x4 wdv = {wd[0], wd[1], wd[2], wd[3]};
      pf[ch] = __builtin_bit_cast(bf16x8, wpv);
      dsf[ch] = __builtin_bit_cast(bf16x8, wdv);
    }

    // the previous stage's dV, dK products (at u = 0 the zero fragments on
    // stage 0's rows, which add exactly nothing)
    dkdv_products(u == 0 ? 0 : (u - 1) % kRing4);
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) {
      // P and dS are needed only by the next iteration: without this use the
      // compiler sinks them past the copies below, out of the products' block
      asm volatile("" ::"v"(pf[ch]), "v"(dsf[ch]));
      pf_prev[ch] = pf[ch];
      dsf_prev[ch] = dsf[ch];
    }

    // stage u + 2 into the slot stage u - 2 used (its last reader, the
    // previous iteration's products, finished before the last barrier);
    // retire stage u + 1
    const bool more = u + 2 < T;
    if (more) copy_stage(u + 2, (u + 2) % kRing4);
    retire(more);
    __syncthreads();
  }
  if (T > 0) dkdv_products((T - 1) % kRing4);

  if (k_ok) {
    __bf16* const dkrow = static_cast<__bf16*>(p.dk) + b * p.k_sb + kvh * p.k_sh + static_cast<size_t>(k_row) * p.k_sr;
    __bf16* const dvrow = static_cast<__bf16*>(p.dv) + b * p.v_sb + kvh * p.v_sh + static_cast<size_t>(k_row) * p.v_sr;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        const u32x2 kk = {pack_bf16(dkt[db][4 * i] * p.scale, dkt[db][4 * i + 1] * p.scale),
                          pack_bf16(dkt[db][4 * i + 2] * p.scale, dkt[db][4 * i + 3] * p.scale)};
        const u32x2 vv = {pack_bf16(dvt[db][4 * i], dvt[db][4 * i + 1]),
                          pack_bf16(dvt[db][4 * i + 2], dvt[db][4 * i + 3])};
        *reinterpret_cast<u32x2*>(dkrow + d0) = kk;
        *reinterpret_cast<u32x2*>(dvrow + d0) = vv;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV at D <= 128 with two waves per SIMD. Eight waves: wave w < 4 and
// wave w + 4 form a pair that owns keys 32 w .. 32 w + 31 of the 128-key
// tile (on the usual round-robin placement both sit on SIMD w). Per 64-row
// query stage u the first wave forms S = Q K^T, P, and dV^T += dO^T P, and
// hands P (times ds'/ds under soft-capping) to its partner through LDS; the
// partner forms dP = dO V^T for stage u and, for stage u - 1 (whose P the
// barrier between the iterations published), dS = P (dP - delta) and
// dK^T += Q^T dS. Each wave holds one of K^T, V^T and one accumulator, so
// both stay within the 256 registers of two waves per SIMD, and one wave's
// exponentials overlap the other's matrix products. Every gradient element
// is still summed by one lane in stage order (no atomics).
// LDS at D = 128: Q ring of three stages (stage u - 1 is read for dK while
// u + 1 arrives), dO ring of two, P in float32 double-buffered, LSE, delta
// and (documents) labels per stage: about 146 KB, one workgroup per CU.
constexpr int kDkv2Threads = 512;
constexpr int kDkvMaxStages = 1024;   // stage list of the document path (Sq up to 64K rows)

template <int D, int MOD, bool DOCS>
__global__ __launch_bounds__(kDkv2Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv2_kernel(BwdLaunch p) {
  static_assert(D == 64 || D == 128, "two-wave dK/dV kernel: D = 64 or 128");
  constexpr int kStage = 64;
  using G = BGeo<D, kStage>;
  constexpr int DC = D / 16, DB = D / 32, RB = G::kRowBytes;
  constexpr int KB = G::kKB, CH = G::kCH;
  constexpr int kQRing = 3, kORing = 2, kSRing = 3;
  // the row's LSE joins the S accumulator's start (the score mod is linear
  // in s; relative bias, also linear, keeps the LSE in the exponent's FMA,
  // since its table lookups leave no registers for the start values)
  constexpr bool kLseInS = MOD == kModNone || MOD == kModAlibi;
  constexpr int kWSlot = 4 * KB * 16 * 64;   // floats of P for the four pairs
  __shared__ __attribute__((aligned(1024))) unsigned char qbuf[kQRing * G::kBufBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char obuf[kORing * G::kBufBytes];
  __shared__ __attribute__((aligned(16))) float wbuf[2 * kWSlot];
  __shared__ __attribute__((aligned(16))) float lbuf[kSRing * kStage];
  __shared__ __attribute__((aligned(16))) float dbuf[kSRing * kStage];
  __shared__ __attribute__((aligned(16))) int labbuf[DOCS ? kSRing * kStage : 4];
  // documents with a block mask: the visited 64-row stages of this key tile
  // in order, (stage << 1) | full, and the class of each candidate 128-row
  // half (0 empty, 1 partial, 3 full)
  __shared__ int slist[DOCS ? kDkvMaxStages : 1];
  __shared__ unsigned char hcls[DOCS ? kDkvMaxStages / 2 + 1 : 1];
  __shared__ int nvis_lds;
  __shared__ float rtab[MOD == kModRelBias ? kRelCap : 1];   // the current head's bias table
  lds_cf32* const tab = (lds_cf32*)(rtab) + p.va.rel_max;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool first = wave < 4;
  const int l32 = lane & 31, g = lane >> 5;

  const int nk = (p.Skv + kRows - 1) / kRows;
  const int total = p.B * p.Hkv * nk;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int lin = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (lin >= total) return;
  const int kt = lin % nk;
  const int bkh = lin / nk;
  const int kvh = bkh % p.Hkv, b = bkh / p.Hkv;
  const int rep = p.H / p.Hkv;
  const unsigned qrb = static_cast<unsigned>(p.q_sr) * 2u, orb = static_cast<unsigned>(p.o_sr) * 2u;
  const unsigned krb = static_cast<unsigned>(p.k_sr) * 2u, vrb = static_cast<unsigned>(p.v_sr) * 2u;

  const int k_row = kt * kRows + pair * 32 + l32;
  const bool k_ok = k_row < p.Skv;

  // the query stages that can see keys [k_lo, k_hi] of this tile (as in the
  // one-wave kernel)
  const bool causal = p.mask_kind & kMaskCausal;
  const bool window = p.mask_kind & kMaskWindow;
  const int off = p.va.q_offset;
  const int k_lo = kt * kRows;
  const int k_hi = min(p.Skv, k_lo + kRows) - 1;
  const int q_first = (causal && k_lo >= p.va.prefix) ? min(max(k_lo - off, 0), p.Sq) : 0;
  const int q_end = window ? static_cast<int>(min(static_cast<long long>(p.Sq),
                                                  static_cast<long long>(k_hi) + p.va.window - off))
                           : p.Sq;
  const int s0 = q_first / kStage;
  const int ns = q_end > q_first ? (q_end + kStage - 1) / kStage - s0 : 0;

  // Under a document mask the block mask (exact per 128-row half and 128-key
  // tile) drops the stages of halves that see none of these keys and marks
  // those that see all of them as full: the lists of the candidate query
  // tiles are read in parallel (one entry per thread), the entries for this
  // key tile give their halves' classes, and wave 0 compacts the visited
  // stages in order. Without a block mask, or past kDkvMaxStages candidate
  // stages, every candidate stage is visited with the mask. The first pass's
  // list lengths and entries are fetched before the K and V rows below, so
  // that the list is in place while those arrive.
  const bool use_list = DOCS && p.kv_count != nullptr && ns > 0 && ns <= kDkvMaxStages;
  const int h0 = s0 >> 1, h1 = (s0 + ns - 1) >> 1;   // candidate halves, inclusive
  const int qp0 = h0 >> 1, nqp = (h1 >> 1) - qp0 + 1;
  const int bm_b = p.bm_num_b > 1 ? b : 0;
  // thread t reads entry j of query tile qp0 + t / 32 + 16 m, j = t % 32 + 32 i
  const int j0 = tid & 31;
  int cnt0 = 0, e00 = 0;
  if (use_list && (tid >> 5) < nqp) {
    const int qp = qp0 + (tid >> 5);
    cnt0 = p.kv_count[bm_b * p.nq + qp];
    e00 = j0 < p.nk ? p.kv_list[(static_cast<size_t>(bm_b) * p.nq + qp) * p.nk + j0] : 0;
  }

  // B operand of this wave's first product: K^T (S = Q K^T) or V^T (dP = dO V^T);
  // lane (key l32, half g) holds 8 consecutive d
  bf16x8 bop[DC];
  {
    const void* base = first ? static_cast<const void*>(static_cast<const __bf16*>(p.k) + b * p.k_sb + kvh * p.k_sh)
                             : static_cast<const void*>(static_cast<const __bf16*>(p.v) + b * p.v_sb + kvh * p.v_sh);
    const unsigned rb = first ? krb : vrb;
    const rsrc_t r = make_rsrc(base, static_cast<unsigned>(p.Skv - 1) * rb + RB);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const unsigned col = (c * 16 + g * 8) * 2;
      const unsigned off = k_ok ? static_cast<unsigned>(k_row) * rb + col : 0x80000000u;
      bop[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
  }
  const int* doc_row = DOCS ? p.va.doc + static_cast<size_t>(b) * p.va.doc_stride : p.va.doc;
  const int doc_k = (DOCS && k_ok) ? doc_row[k_row] : 0;


  int nvis = ns;
  if constexpr (DOCS) {
    if (use_list) {
      for (int i = tid; i <= h1 - h0; i += kDkv2Threads) hcls[i] = 0;
      __syncthreads();
      auto note = [&](int qp, int e) {
        if ((e >> 4) == kt) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int h = 2 * qp + hf;
            if (h >= h0 && h <= h1) hcls[h - h0] = static_cast<unsigned char>((e >> (2 * hf)) & 3);
          }
        }
      };
      for (int m = 0; m * 16 < nqp; ++m) {
        const int qp = qp0 + m * 16 + (tid >> 5);
        if (qp - qp0 < nqp) {
          const int* lst = p.kv_list + (static_cast<size_t>(bm_b) * p.nq + qp) * p.nk;
          const int cnt = m == 0 ? cnt0 : p.kv_count[bm_b * p.nq + qp];
          const int e0 = m == 0 ? e00 : (j0 < p.nk ? lst[j0] : 0);
          if (j0 < cnt) note(qp, e0);
          for (int j = j0 + 32; j < cnt; j += 32) note(qp, lst[j]);
        }
      }
      __syncthreads();
      if (wave == 0) {
        int base = 0;
        for (int j0 = 0; j0 < ns; j0 += 64) {
          const int j = j0 + lane;
          const int c = j < ns ? hcls[((s0 + j) >> 1) - h0] : 0;
          const uint64_t m = __builtin_amdgcn_ballot_w64(c != 0);
          const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(m), 0));
          if (c != 0) slist[base + rank] = ((s0 + j) << 1) | (c == 3 ? 1 : 0);
          base += __builtin_popcountll(m);
        }
        if (lane == 0) nvis_lds = base;
      }
      __syncthreads();
      nvis = __builtin_amdgcn_readfirstlane(nvis_lds);
    }
  }
  const int T = rep * nvis;
  // stage u: query head kvh rep + u / nvis; (64-row stage << 1) | full
  auto stage_of = [&](int u) -> int {
    const int j = u % nvis;
    if constexpr (DOCS) {
      if (use_list) return __builtin_amdgcn_readfirstlane(slist[j]);
    }
    return (s0 + j) << 1;
  };

  // fragment offsets from one base each: the chunk permutation touches only
  // the low chunk bits and a row's chunk bits sit below its row offset, so
  // chunk 2c + g's row offset is chunk g's XOR 32 c and block db's
  // transposed offset block 0's XOR 64 db (at D = 64 and 128 alike)
  const unsigned qoff0 = row_off<D>(l32, g);
  const unsigned toff0[2] = {trans_off<D>(lane, 0, 0), trans_off<D>(lane, 0, 1)};
  auto qoff = [&](int c) -> unsigned { return qoff0 ^ static_cast<unsigned>(c << 5); };
  auto toff = [&](int db, int j) -> unsigned { return toff0[j] ^ static_cast<unsigned>(db << 6); };

  const unsigned ql = lds_addr(qbuf), ol = lds_addr(obuf);
  const unsigned ll = lds_addr(lbuf), dl = lds_addr(dbuf), labl = lds_addr(labbuf);
  // all eight waves share the tile copies of stage u, wave 0 copies LSE and
  // delta and wave 1 the rows' document labels
  auto copy_stage = [&](int u) {
    const int hh = kvh * rep + u / nvis;
    const int r0 = (stage_of(u) >> 1) * kStage;
    const u32x4 qd = make_desc(static_cast<const __bf16*>(p.q) + b * p.q_sb + hh * p.q_sh,
                               static_cast<unsigned>(p.Sq - 1) * qrb + RB);
    const u32x4 od = make_desc(static_cast<const __bf16*>(p.dout) + b * p.o_sb + hh * p.o_sh,
                               static_cast<unsigned>(p.Sq - 1) * orb + RB);
    copy_tile<D, kStage, 8>(qd, static_cast<unsigned>(r0) * qrb, qrb, ql + (u % kQRing) * G::kBufBytes, wave, lane);
    copy_tile<D, kStage, 8>(od, static_cast<unsigned>(r0) * orb, orb, ol + (u % kORing) * G::kBufBytes, wave, lane);
    const int sl = u % kSRing;
    if (wave == 0 && lane < kStage / 4) {
      const size_t q_head = (static_cast<size_t>(b) * p.H + hh) * p.Sq;
      const u32x4 lsd = make_desc(p.lse + q_head, static_cast<unsigned>(p.Sq) * 4u);
      const u32x4 dld = make_desc(p.delta + q_head, static_cast<unsigned>(p.Sq) * 4u);
      copy_to_lds(lsd, static_cast<unsigned>(r0) * 4u + lane * 16u, __builtin_amdgcn_readfirstlane(ll + sl * kStage * 4));
      copy_to_lds(dld, static_cast<unsigned>(r0) * 4u + lane * 16u, __builtin_amdgcn_readfirstlane(dl + sl * kStage * 4));
    }
    if constexpr (DOCS) {
      if (wave == 1 && lane < kStage / 4) {
        // positions past the label array read as zero; their rows are past
        // Sq and masked by the query range
        const u32x4 ld = make_desc(doc_row, static_cast<unsigned>(p.va.doc_stride) * 4u);
        copy_to_lds(ld, static_cast<unsigned>(r0 + off) * 4u + lane * 16u,
                    __builtin_amdgcn_readfirstlane(labl + sl * kStage * 4));
      }
    }
  };
  // a new query head under relative bias: its table replaces the last
  // head's, whose last reader (the previous stage's P) finished before the
  // previous barrier; every wave takes this barrier
  auto head_table = [&](int u) {
    if constexpr (MOD == kModRelBias) {
      if (u % nvis == 0) {
        stage_rel_table(p.va, kvh * rep + u / nvis, (lds_f32*)(rtab), tid, kDkv2Threads);
        __syncthreads();
      }
    }
  };

  if (T > 0) copy_stage(0);
  wait_vm<0>();
  __syncthreads();

  f32x16 acc[DB];   // dV^T (first wave) or dK^T (second)
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  if (first) {
    for (int u = 0; u < T; ++u) {
      head_table(u);
      if (u + 1 < T) copy_stage(u + 1);
      const int hh = __builtin_amdgcn_readfirstlane(kvh * rep + u / nvis);
      const int st = stage_of(u);
      const int r0 = (st >> 1) * kStage;
      const unsigned char* qb_ = qbuf + (u % kQRing) * G::kBufBytes;
      const unsigned char* ob_ = obuf + (u % kORing) * G::kBufBytes;
      const float* lb = lbuf + (u % kSRing) * kStage;
      const int q_last = r0 + kStage - 1;
      // every pair of the stage in range and admitted? (for documents the
      // block mask's class, which accounts for every part of the mask)
      bool full = !DOCS && q_last < p.Sq && k_hi == k_lo + kRows - 1;
      if (causal) full = full && (r0 + off >= k_hi || k_hi < p.va.prefix);
      if (window) full = full && (q_last + off - k_lo < p.va.window);
      if (DOCS && use_list) full = (st & 1) != 0;
      float slope2 = 0.f;
      if constexpr (MOD == kModAlibi) {
        // a scalar load (constant address space, uniform index): a vector
        // load's wait would also wait for the copies just issued
        const __attribute__((address_space(4))) float* sl =
            (const __attribute__((address_space(4))) float*)(p.va.slopes);
        slope2 = sl[hh] * kLog2e;
      }

      // S = Q K^T: KB 32-row query blocks, each operand read issued four
      // products ahead of its product (the compiler's own order waits on
      // almost every read). Without a score mod and under ALiBi (linear in
      // s) the row's LSE goes into the accumulator's start,
      // -LSE log2(e) / c1, so the modified score is already t - log2(e) LSE.
      // A row with no admitted key (LSE = -inf) starts at +inf; it lies in
      // partial stages only, whose mask sets every one of its scores to -inf.
      f32x16 s[KB];
      if constexpr (kLseInS) {
        const float f = -kLog2e / p.va.c1;
#pragma unroll
        for (int qb = 0; qb < KB; ++qb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lb + 32 * qb + 8 * i4 + 4 * g);
#pragma unroll
            for (int x = 0; x < 4; ++x) s[qb][4 * i4 + x] = l4[x] * f;
          }
      } else {
#pragma unroll
        for (int qb = 0; qb < KB; ++qb) s[qb] = f32x16{};
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int qb = 0; qb < KB; ++qb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(qb_ + qoff(c) + qb * 32 * RB);
          s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[c], s[qb], 0, 0, 0);
        }
      reads_ahead<DC * KB, 4, 1>();

      // modified scores, masked in place on partial stages (element 16 qb + i
      // is row r0 + 32 qb + 8 (i / 4) + 4 g + i % 4)
      float tt[KB * 16];
      float dmv[MOD == kModSoftcap ? KB * 16 : 1];
#pragma unroll
      for (int qb = 0; qb < KB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qpos = r0 + 32 * qb + 8 * (i >> 2) + 4 * g + (i & 3) + off;
          float dmod;
          tt[qb * 16 + i] = mod_score<MOD>(s[qb][i], p.va, slope2, tab, k_row - qpos, dmod);
          if constexpr (MOD == kModSoftcap) dmv[qb * 16 + i] = dmod;
        }
      if (!full) {
        const float ninf = -INFINITY;
        const int rr0 = r0 + 4 * g;
        const long long kq = static_cast<long long>(k_row) - off - rr0;
        long long hi = static_cast<long long>(p.Sq) - 1 - rr0;
        if (window) hi = min(hi, kq + p.va.window - 1);
        if (!k_ok) hi = -1;
        const long long lo = (causal && k_row >= p.va.prefix) ? kq : 0LL;
        int hi_c = static_cast<int>(min(max(hi, -1LL), static_cast<long long>(kStage)));
        const int lo_c = static_cast<int>(min(max(lo, 0LL), static_cast<long long>(kStage)));
        bool need_doc = false;
        const int* lab = labbuf + (u % kSRing) * kStage;
        if constexpr (DOCS) {
          const int lq = lab[lane & (kStage - 1)];
          const int l0 = __builtin_amdgcn_readfirstlane(lq);
          if (__all(lq == l0)) {
            if (doc_k != l0) hi_c = -1;
          } else {
            need_doc = true;
          }
        }
        if (need_doc) {
#pragma unroll
          for (int qb = 0; qb < KB; ++qb)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int4 l4 = *reinterpret_cast<const int4*>(lab + 32 * qb + 8 * i4 + 4 * g);
              const int lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
              for (int x = 0; x < 4; ++x)
                mask_in_place(tt[qb * 16 + 4 * i4 + x], __builtin_amdgcn_ballot_w64(lv[x] == doc_k), ninf);
            }
        }
        if (!__all(lo_c <= 0)) {
#pragma unroll
          for (int j = 0; j < KB * 16; ++j)
            mask_in_place(tt[j], __builtin_amdgcn_ballot_w64((j >> 4) * 32 + 8 * ((j >> 2) & 3) + (j & 3) >= lo_c),
                          ninf);
        }
        if (!__all(hi_c >= kStage - 1)) {
#pragma unroll
          for (int j = 0; j < KB * 16; ++j)
            mask_in_place(tt[j], __builtin_amdgcn_ballot_w64((j >> 4) * 32 + 8 * ((j >> 2) & 3) + (j & 3) <= hi_c),
                          ninf);
        }
      }

      // P = exp2(t - log2(e) LSE) (where the LSE is not in S, it is clamped
      // by one med3 so that a row with no admitted key gives P = 0, not NaN);
      // P, times ds'/ds under soft-capping, goes to the partner as float32,
      // P as bf16 into the B operand of dV^T += dO^T P
      float* wout = wbuf + (u & 1) * kWSlot + pair * (KB * 16 * 64);
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int qb = ch >> 1, i0 = (ch & 1) * 8;
        unsigned wp[4];
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          f32x4 pv;
          if constexpr (kLseInS) {
#pragma unroll
            for (int x = 0; x < 4; ++x) pv[x] = __builtin_amdgcn_exp2f(tt[qb * 16 + i0 + 4 * hv + x]);
          } else {
            const int ql0 = 32 * qb + 8 * ((i0 >> 2) + hv) + 4 * g;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lb + ql0);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const float lc = __builtin_amdgcn_fmed3f(l4[x], -1e30f, 3e38f);
              pv[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(lc, -kLog2e, tt[qb * 16 + i0 + 4 * hv + x]));
            }
          }
          f32x4 wv = pv;
          if constexpr (MOD == kModSoftcap) {
#pragma unroll
            for (int x = 0; x < 4; ++x) wv[x] *= dmv[qb * 16 + i0 + 4 * hv + x];
          }
          *reinterpret_cast<f32x4*>(wout + ((2 * ch + hv) * 64 + lane) * 4) = wv;
          wp[2 * hv] = pack_bf16(pv[0], pv[1]);
          wp[2 * hv + 1] = pack_bf16(pv[2], pv[3]);
        }
        const u32x4 wpv = {wp[0], wp[1], wp[2], wp[3]};
        const bf16x8 pf = __builtin_bit_cast(bf16x8, wpv);
        // dV^T += dO^T P for this chunk of 16 rows (each accumulator still
        // sums the chunks in order)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(trans_frag<D>(ob_, toff(db, 0), toff(db, 1), ch), pf,
                                                            acc[db], 0, 0, 0);
      }
      wait_vm<0>();
      __syncthreads();
    }
  } else {
    // dS of stage v from its P (published by the barrier that ended
    // iteration v) and dP, packed to bf16 in the key order of the B operand
    // (delta subtracted after the products, so that dP - delta cancels
    // exactly where P = 1, as in the dQ kernel)
    auto ds_of = [&](int v, const f32x16 (&dp)[KB], bf16x8 (&dsf)[CH]) {
      const float* win = wbuf + (v & 1) * kWSlot + pair * (KB * 16 * 64);
      const float* dlb = dbuf + (v % kSRing) * kStage;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int qb = ch >> 1, i0 = (ch & 1) * 8;
        unsigned wd[4];
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          const f32x4 wv = *reinterpret_cast<const f32x4*>(win + ((2 * ch + hv) * 64 + lane) * 4);
          float dv4[4];
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlb + 32 * qb + 8 * ((i0 >> 2) + hv) + 4 * g);
#pragma unroll
          for (int x = 0; x < 4; ++x) dv4[x] = wv[x] * (dp[qb][i0 + 4 * hv + x] - d4[x]);
          wd[2 * hv] = pack_bf16(dv4[0], dv4[1]);
          wd[2 * hv + 1] = pack_bf16(dv4[2], dv4[3]);
        }
        const u32x4 wdv = {wd[0], wd[1], wd[2], wd[3]};
        dsf[ch] = __builtin_bit_cast(bf16x8, wdv);
      }
    };
    // dK^T += Q^T dS of stage v, product i (chunk i / DB, block i % DB:
    // each accumulator sums the chunks in order)
    auto dk_product = [&](int v, int i, const bf16x8 (&dsf)[CH]) {
      const unsigned char* qp_ = qbuf + (v % kQRing) * G::kBufBytes;
      const int ch = i / DB, db = i % DB;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(trans_frag<D>(qp_, toff(db, 0), toff(db, 1), ch), dsf[ch],
                                                        acc[db], 0, 0, 0);
    };
    // dP = dO V^T of stage u, product i (d chunk i / KB, row block i % KB)
    auto dp_product = [&](int u, int i, f32x16 (&dp)[KB]) {
      const unsigned char* ob_ = obuf + (u % kORing) * G::kBufBytes;
      const int c = i / KB, qb = i % KB;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(ob_ + qoff(c) + qb * 32 * RB);
      dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[c], dp[qb], 0, 0, 0);
    };
    constexpr int NPROD = DC * KB;   // dP products per stage; as many dK products
    static_assert(NPROD == CH * DB, "product counts");
    // one iteration: dS and dK of stage u - 1, which consume dP of stage
    // u - 1, then dP of stage u into the same registers. The dS work needs
    // nothing from this iteration, so it runs while the first wave's S
    // products occupy the matrix unit, and the dK and dP products then run
    // beside the first wave's exponentials.
    f32x16 dp[KB];
    bf16x8 dsf[CH];
    for (int u = 0; u < T; ++u) {
      head_table(u);
      if (u + 1 < T) copy_stage(u + 1);
      if (u > 0) ds_of(u - 1, dp, dsf);
#pragma unroll
      for (int qb = 0; qb < KB; ++qb) dp[qb] = f32x16{};
      __builtin_amdgcn_sched_barrier(0);
      if (u > 0) {
        // dK products of stage u - 1 and dP products of stage u alternate
        // (two independent chains), operand reads three pairs ahead
#pragma unroll
        for (int i = 0; i < NPROD; ++i) {
          dk_product(u - 1, i, dsf);
          dp_product(u, i, dp);
        }
        reads_ahead<NPROD, 3, 3>();
      } else {
#pragma unroll
        for (int i = 0; i < NPROD; ++i) dp_product(u, i, dp);
        reads_ahead<NPROD, 4, 1>();
      }
      wait_vm<0>();
      __syncthreads();
    }
    if (T > 0) {
      ds_of(T - 1, dp, dsf);
#pragma unroll
      for (int i = 0; i < NPROD; ++i) dk_product(T - 1, i, dsf);
    }
  }

  if (k_ok) {
    const float sc = first ? 1.f : p.scale;
    __bf16* const row = first
        ? static_cast<__bf16*>(p.dv) + b * p.v_sb + kvh * p.v_sh + static_cast<size_t>(k_row) * p.v_sr
        : static_cast<__bf16*>(p.dk) + b * p.k_sb + kvh * p.k_sh + static_cast<size_t>(k_row) * p.k_sr;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        const u32x2 vv = {pack_bf16(acc[db][4 * i] * sc, acc[db][4 * i + 1] * sc),
                          pack_bf16(acc[db][4 * i + 2] * sc, acc[db][4 * i + 3] * sc)};
        *reinterpret_cast<u32x2*>(row + d0) = vv;
      }
  }
}

template <int D, int MOD, bool DOCS>
hipError_t launch_t(const BwdLaunch& p, hipStream_t stream) {
  {
    const long long total = static_cast<long long>(p.B) * p.H * ((p.Sq + kRows - 1) / kRows);
    const long long per = (total + kXcds - 1) / kXcds;
    note_launch("attn_bwd_dq_kernel<%d, %d, %s> grid %lld x %d", D, MOD, DOCS ? "true" : "false", per * kXcds,
                kThreads);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, MOD, DOCS>), dim3(static_cast<unsigned>(per * kXcds)),
                       dim3(kThreads), 0, stream, p, p.kv_count, p.kv_list);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long total = static_cast<long long>(p.B) * p.Hkv * ((p.Skv + kRows - 1) / kRows);
  const long long per = (total + kXcds - 1) / kXcds;
  if constexpr (D <= 128) {
    note_launch("attn_bwd_dkdv2_kernel<%d, %d, %s> grid %lld x %d", D, MOD, DOCS ? "true" : "false", per * kXcds,
                kDkv2Threads);
    hipLaunchKernelGGL((attn_bwd_dkdv2_kernel<D, MOD, DOCS>), dim3(static_cast<unsigned>(per * kXcds)),
                       dim3(kDkv2Threads), 0, stream, p);
  } else {
    note_launch("attn_bwd_dkdv_kernel<%d, %d, %s> grid %lld x %d", D, MOD, DOCS ? "true" : "false", per * kXcds,
                kThreads);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, MOD, DOCS>), dim3(static_cast<unsigned>(per * kXcds)),
                       dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <int D, bool DOCS>
hipError_t launch_mod(const BwdLaunch& p, hipStream_t stream) {
  switch (p.mod_kind) {
    case kModNone: return launch_t<D, kModNone, DOCS>(p, stream);
    case kModAlibi: return launch_t<D, kModAlibi, DOCS>(p, stream);
    case kModSoftcap: return launch_t<D, kModSoftcap, DOCS>(p, stream);
    case kModRelBias: return launch_t<D, kModRelBias, DOCS>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_bwd(const BwdLaunch& p, hipStream_t stream) {
  if (p.nk > kPairMaxKeyTiles) return hipErrorInvalidValue;
  const bool docs = p.mask_kind & kMaskDocument;
  if (p.D == 256) return docs ? launch_mod<256, true>(p, stream) : launch_mod<256, false>(p, stream);
  if (p.D == 128) return docs ? launch_mod<128, true>(p, stream) : launch_mod<128, false>(p, stream);
  if (p.D == 64) return docs ? launch_mod<64, true>(p, stream) : launch_mod<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
