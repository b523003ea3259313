// attn_fwd_pp.hip - bf16 attention forward for gfx950 (MI355X, CDNA4): 256-row
// workgroups of two wave groups that run in ping-pong.
//
// What is computed is the fused, tiled forward of attn_fwd.hip (online softmax
// over key tiles kept on chip, no approximation: Neuron FA4 explainer, "Enter
// Tri Dao and FlashAttention"). This kernel adds the scheduling idea of the
// FA4 forward-pass fixes (same page, "FlashAttention-4: Built for Blackwell"):
// two independent sets of query rows alternate, so that while one set runs its
// matrix products the other runs its exponentials.
//
// Mapping to CDNA4:
//  * A workgroup of 8 waves owns 256 query rows of one (batch, head). Waves
//    0-3 (group 0) take rows 0-127, waves 4-7 (group 1) rows 128-255; wave w
//    and wave w + 4 share a SIMD. Each wave owns 32 rows.
//  * Time runs in barrier-separated slots. A group alternates a matrix slot,
//    S^T(t) = K(t) Q^T and O^T += V(t-1)^T P^T(t-1) (32 v_mfma_f32_32x32x16_bf16
//    per wave at D = 128), with a vector slot: the online softmax of stage t.
//    Group 1 runs one slot behind group 0, so every SIMD always has one wave
//    multiplying and one exponentiating. Both groups run the same code; the
//    offset is one extra barrier at the start (group 1) and at the end
//    (group 0). At D = 256 (32-key stages, half the softmax per slot) the
//    groups run in phase instead.
//  * Both groups read the same K and V stage buffers, so each tile is brought
//    on chip once per 256 query rows. Group 0 loads K, group 1 loads V, each
//    in its vector slot and two stages ahead, as direct buffer-to-LDS copies:
//    no registers, no VALU work, and a ring of three stage buffers.
//  * V stays row-major in LDS. The A operand of O^T += V^T P^T (32 values of
//    d, 8 keys per lane) comes from two ds_read_b64_tr_b16 per fragment: each
//    16-lane group of that instruction turns a 4-key x 16-d block into one
//    d column of 4 keys per lane.
//  * K and V rows are unpadded; 16-byte chunks are XOR-permuted by row so that
//    the fragment reads of both products are free of bank conflicts and every
//    1 KB copy lands in one contiguous LDS run (lane i writes slot i).
//  * The S^T accumulator layout gives each lane 32 scores of one query row:
//    the row max is one permlane32 swap, the running sum stays lane-local, and
//    the accumulators rounded to bf16 are directly the B operand P^T.
//  * Conditional rescaling with a threshold of 2^8 (same forward-pass fixes),
//    scale folded into exp2, XCD-aware and heavy-first tile order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_util.h"
#include "exp2_poly.h"
#include "launch.h"
#include "variants.h"

// Share of the softmax exponentials evaluated by the polynomial of
// exp2_poly.h instead of the hardware unit: the first N 16-key chunks of
// each stage (a build option, 0 by default: measured slower, since the vector
// slot is bound by the issue rate of one wave, where a polynomial costs about
// eight instructions against one).
#ifndef FLEXATTN_EXP2_POLY_CHUNKS
#define FLEXATTN_EXP2_POLY_CHUNKS 0
#endif

// Every fused multiply-add of this file is written out (__builtin_fmaf), so
// the compiler may not fuse others: a copy of the loop it specialises (the
// first stage, where the exponent base is a known zero) would otherwise round
// some scores differently from the loop body, and whether a stage takes the
// specialised copy depends on how many empty stages precede it.
#pragma clang fp contract(off)

namespace fa {
namespace {

using namespace dev;

constexpr int kThreads = 512;   // 8 waves: two groups of 4
constexpr int kBM = 2 * kPairHalf;   // query rows per workgroup
constexpr int kBNMax = 64;      // keys per stage (32 at D = 256)
constexpr int kTile = 128;      // key tile of the block mask
constexpr int kRing = 3;        // stage buffers for K and for V
constexpr int kXcds = 8;
constexpr int kLptMaxTiles = 256;   // longest-first order up to this many query tiles
constexpr float kRescaleLog2 = 8.0f;
constexpr float kSumLimit = 256.0f;   // 2^kRescaleLog2

template <int D>
struct PGeo {
  // keys per stage: 64, or 32 at D = 256 so that a K or V stage stays 16 KB
  static constexpr int kBN = D == 256 ? 32 : 64;
  static constexpr int kKB = kBN / 32;                 // 32-key blocks of S^T
  static constexpr int kCH = kBN / 16;                 // 16-key chunks of P^T
  static constexpr int kSPT = 128 / kBN;               // stages per 128-key tile
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBufBytes = kBN * D * 2;        // one K or V stage
  static constexpr int kCpr = D / 8;                   // 16-byte chunks per row
  static constexpr int kDma = kBufBytes / 1024 / 4;    // 1 KB copies per wave of a group
  static_assert(kDma >= 1 && kBufBytes % 4096 == 0, "stage geometry");
};

// Chunk permutations (chunk c of row r sits at position c ^ swz(r)). K: the
// 16 rows read together by one quarter-wave of a b128 fragment read hit 16
// different chunk positions. V: the 4 rows read together by one half-wave of
// a transposing b64 read hit disjoint groups of 4 chunks.
template <int D>
__device__ inline int kswz(int r) { return D == 256 ? r % 16 : (r / (128 / D)) % (D / 8); }
template <int D>
__device__ inline int vswz(int r) { return D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// PACK (decode mode): a workgroup owns the rep = H / Hkv query heads of one
// key/value head, packed as rows r = head_in_group * Sq + q_row (at most 256),
// and one of p.splits contiguous parts of the key-tile list of query tile 0.
// Without PACK, p.splits > 1 cuts every query tile's list the same way. Split
// results go to the workspace and attn_decode_merge_kernel combines them.
// Waves per SIMD: 2 (one workgroup per CU), or 4 (two workgroups per CU) at
// D = 64, where a wave fits 128 registers and a workgroup ~57 KB of LDS. There
// the softmax outweighs the products, and the other workgroup's waves add
// vector issue slots (A/B on one machine: alibi_d64 +12%, softcap_d64 +18%, doc_swa
// at D = 64 +29%, dense at D = 64 +6%). Not with the relative-bias table or in
// decode mode, whose registers do not fit 128 without spilling (6% and 11%
// slower measured).
template <int D, int MOD, int PACK>
constexpr int kWavesPerSimd = (D == 64 && PACK == 0 && MOD != kModRelBias) ? 4 : 2;

// PACK: 0 the regular mapping; 1 decode mode; 2 decode mode with at most 128
// packed rows (D <= 128); 3 the regular mapping when Sq <= 128 (D <= 128).
// In modes 2 and 3 (key split) the rows sit in the waves of both groups
// alike: wave w of group 0 and wave w of group 1 (one SIMD) hold the same 32
// rows and each takes one 32-key half of every stage with a running softmax
// of its own; the two are merged once after the loop. One wave's products
// then overlap its partner's softmax, where with the rows in one group a
// stage costs each wave's matrix and vector work back to back (and, in the
// regular mapping, the other group works on padding rows).
template <int D, int MOD, bool DOCS, int PACK>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D, MOD, PACK>, kWavesPerSimd<D, MOD, PACK>)))
void attn_fwd_pp_kernel(FwdLaunch p, const int* __restrict__ kv_count, const int* __restrict__ kv_list) {
  using G = PGeo<D>;
  constexpr bool KS = PACK == 2 || PACK == 3;   // key halves split between the groups
  constexpr bool PK = PACK == 1 || PACK == 2;   // packed rows (decode mode)
  static_assert(!KS || D <= 128, "key split needs 64-key stages");
  constexpr int DC = D / 16;   // 16-wide d chunks (k-steps of S^T)
  constexpr int DB = D / 32;   // 32-row d blocks of O^T
  constexpr int RB = G::kRowBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[kRing * G::kBufBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[kRing * G::kBufBytes];
  __shared__ int ents[kPairMaxKeyTiles];
  // document labels of each ring slot's 64 keys (copied with K by wave 0)
  __shared__ __attribute__((aligned(16))) int labbuf[DOCS ? kRing * kBNMax : 4];
  __shared__ float rtab[MOD == kModRelBias ? kRelCap : 1];   // this head's bias table

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int wq = wave & 3;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- workgroup -> (b, h, 256-row tile[, split]): XCD-contiguous, heavy
  // tiles first; decode mode: (b, key/value head, split)
  const int rep = p.H / p.Hkv;
  const int np = PK ? 1 : (p.Sq + kBM - 1) / kBM;
  const int total = (PK ? p.B * p.Hkv : p.B * p.H * np) * p.splits;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int wg = blockIdx.x;
  const int lin = (wg % kXcds) * per_xcd + wg / kXcds;
  if (lin >= total) return;
  // split-KV (p.splits > 1): the splits of one item are consecutive
  const int split = lin % p.splits;
  const int item = lin / p.splits;
  int qp = PK ? 0 : np - 1 - (item % np);
  int slice = item / np;   // (b, h) of the regular kernel
  // length and first entry of the item's key-tile list when the mapping
  // below has fetched them (n_head < 0: not fetched)
  int n_head = -1, e_head = 0;
  if constexpr (DOCS && !PK) {
    // Document masks make the work of a slice's query tiles uneven. When the
    // slices split evenly over the XCDs, each XCD takes its slices' items
    // longest first (most key tiles; ties: the later tile), rank-major over
    // its slices, so the 32 CUs of an XCD finish together. Every item is
    // computed the same way whichever workgroup takes it. The first entry of
    // every tile's list is fetched with the counts, so the chosen item's
    // first copies need no further round trip.
    const int spx = p.B * p.H / kXcds;
    if (kv_count && p.splits == 1 && p.nq <= kLptMaxTiles && spx * kXcds == p.B * p.H) {
      __shared__ int sel[3];
      const int j = wg / kXcds;
      const int rank = j / spx;
      slice = (wg % kXcds) * spx + j % spx;
      const int row0 = (p.bm_num_b > 1 ? slice / p.H : 0) * p.nq;
      int* const keys = ents;                  // staged before the key-tile list
      int* const heads = ents + kLptMaxTiles;
      if (tid < p.nq) {
        const int c = kv_count[row0 + tid];
        heads[tid] = kv_list[static_cast<size_t>(row0 + tid) * p.nk];   // slot 0 exists (nk >= 1)
        keys[tid] = c * 65536 + tid;
      }
      if (tid == 0) sel[0] = sel[1] = sel[2] = 0;
      __syncthreads();
      if (tid < p.nq) {
        const int mine = keys[tid];
        int above = 0;
        for (int i = 0; i < p.nq; ++i) above += keys[i] > mine;
        if (above == rank) {
          sel[0] = tid;
          sel[1] = mine >> 16;
          sel[2] = heads[tid];
        }
      }
      __syncthreads();
      qp = min(max(__builtin_amdgcn_readfirstlane(sel[0]), 0), np - 1);
      n_head = min(max(__builtin_amdgcn_readfirstlane(sel[1]), 0), p.nk);
      e_head = __builtin_amdgcn_readfirstlane(sel[2]);
      __syncthreads();   // the keys are read before the list overwrites them
    }
  }
  const int b = PK ? item / p.Hkv : slice / p.H;
  const int kvh = PK ? item % p.Hkv : (slice % p.H) / rep;
  // this lane's row: packed index r (decode mode), its query head and row
  const int r_lane = (KS ? 0 : grp * kPairHalf) + wq * 32 + l32;
  const int hl = PK ? min(r_lane / p.Sq, rep - 1) : 0;
  const int h = PK ? kvh * rep + hl : slice % p.H;   // lane-varying in decode mode
  const int q_row = PK ? r_lane - hl * p.Sq : qp * kBM + r_lane;
  const bool q_ok = PK ? r_lane < rep * p.Sq : q_row < p.Sq;
  // decode mode: a wave whose 32 rows all lie past the packed rows only
  // copies and keeps the barriers (wave-uniform, fixed for the whole loop)
  const bool live = PACK == 3 ? __builtin_amdgcn_readfirstlane(q_row - l32) < p.Sq
                               : !PK || __builtin_amdgcn_readfirstlane(r_lane - l32) < rep * p.Sq;
  const size_t q_head = (static_cast<size_t>(b) * p.H + h) * p.Sq;   // LSE rows
  // row strides in bytes; a (batch, head) slice spans rows 0 .. S - 1, so
  // rows past the end read as zero (decode mode: the slices of the group's
  // heads, from its first head)
  const unsigned qrb = static_cast<unsigned>(p.q_sr) * 2u;
  const unsigned grb = static_cast<unsigned>(grp ? p.v_sr : p.k_sr) * 2u;   // this group's K or V
  const __bf16* qbase = static_cast<const __bf16*>(p.q) + b * p.q_sb + (PK ? kvh * rep : h) * p.q_sh;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + b * p.k_sb + kvh * p.k_sh;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + b * p.v_sb + kvh * p.v_sh;
  const unsigned q_bytes = PK ? static_cast<unsigned>((rep - 1) * p.q_sh * 2 + (p.Sq - 1) * qrb + RB)
                                : static_cast<unsigned>(p.Sq - 1) * qrb + RB;
  const rsrc_t rq = make_rsrc(qbase, q_bytes);
  const unsigned kv_bytes = static_cast<unsigned>(p.Skv - 1) * grb + RB;
  const u32x4 desc = grp ? make_desc(vbase, kv_bytes) : make_desc(kbase, kv_bytes);

  // ---- key-tile list of this 256-row tile. Entry:
  // (kv_tile << 4) | full1 << 3 | any1 << 2 | full0 << 1 | any0 (half 0 = rows
  // 0-127 of the tile, half 1 = rows 128-255). No block mask: every tile,
  // both halves partial. Its length and first entry are read first (beside
  // the Q loads), so that the first two stages' copies start one memory
  // round trip after entry; the row holds nk slots, so its first kThreads
  // entries are read at the same time.
  const int bm_b = (kv_count && p.bm_num_b > 1) ? b : 0;
  const int* list = kv_count ? kv_list + (static_cast<size_t>(bm_b) * p.nq + qp) * p.nk : nullptr;
  int n_entries = p.nk;
  int e_spec = 0;
  // Key order. ALiBi's bias grows with the key position, so under a causal
  // mask ascending keys would raise the running max past the rescale
  // threshold (and rescale O) on most stages of most heads; visiting the key
  // tiles in descending order meets the largest biases first, after which the
  // farther keys only score lower. Other variants take ascending order.
  constexpr bool kDesc = MOD == kModAlibi;
  // the whole list, from its head: the first copies start before it is
  // staged (ascending order only: the descending order starts at its tail)
  const bool early = !PK && p.splits == 1 && !kDesc;
  if (!early || n_head < 0) {
    if (kv_count) n_entries = kv_count[bm_b * p.nq + qp];
    if (early && list) {
      e_head = list[0];
      if (tid < p.nk) e_spec = list[tid];
    }
  } else {
    n_entries = n_head;
  }
  // Without a block mask a key tile is partial (every element tested), except
  // when there is no mask at all: then a tile wholly inside Skv is full.
  auto unlisted = [&](int j) -> int {
    return (j << 4) | ((p.mask_kind == 0 && (j + 1) * kTile <= p.Skv) ? 0xF : 0x5);
  };
  if (!list) e_head = unlisted(0);

  // Q^T fragments (B operand of S^T): rows past Sq (and, in decode mode,
  // packed rows past the group) read as zero
  const unsigned q_off = !q_ok ? 0x80000000u
                         : PK ? static_cast<unsigned>(hl * p.q_sh * 2) + static_cast<unsigned>(q_row) * qrb
                                : static_cast<unsigned>(q_row) * qrb;
  bf16x8 qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c)
    qf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
        rq, q_off + (c * 16 + g * 8) * 2, 0, 0));

  constexpr int kBN = G::kBN, kSPT = G::kSPT;
  auto stage_kv0 = [](int t, int e) -> int { return (e >> 4) * kTile + (t % kSPT) * kBN; };

  // ---- per-lane LDS offsets
  // K fragment (S^T A operand): row l32 (+32 kb), chunk 2c + g
  // (at D = 256 the offsets are formed as needed: the chunk permutation is an
  // XOR of low bits, so chunk c's offset is the chunk-0 offset XOR 32 c, and
  // block db's V offset the block-0 offset XOR 64 db; this saves 23 registers)
  constexpr bool kXorOff = D == 256;
  unsigned koff[kXorOff ? 1 : DC];
#pragma unroll
  for (int c = 0; c < (kXorOff ? 1 : DC); ++c) koff[c] = l32 * RB + (((2 * c + g) ^ kswz<D>(l32)) * 16);
  auto koff_at = [&](int c) -> unsigned { return kXorOff ? koff[0] ^ (c << 5) : koff[c]; };
  // V^T fragment via transposing reads: 16-lane group G, lane sl reads 4 d
  // values of key row 16 ch + 8 j + 4 (G / 2) + sl / 4 starting at
  // d = 32 db + 16 (G % 2) + 4 (sl % 4)
  unsigned voff[kXorOff ? 1 : DB];
  {
    const int G16 = lane >> 4, sl = lane & 15;
    const int row0 = 4 * (G16 >> 1) + (sl >> 2);
#pragma unroll
    for (int db = 0; db < (kXorOff ? 1 : DB); ++db) {
      const int chunk = 4 * db + 2 * (G16 & 1) + ((sl & 3) >> 1);
      voff[db] = row0 * RB + ((chunk ^ vswz<D>(row0)) * 16) + (sl & 1) * 8;
    }
  }
  auto voff_at = [&](int db) -> unsigned { return kXorOff ? voff[0] ^ (db << 6) : voff[db]; };
  // copies: this wave fills 1 KB runs wq * kDma + j of a stage buffer; lane i
  // writes slot i of the run, i.e. chunk position s % kCpr of row s / kCpr
  unsigned goff[G::kDma];
#pragma unroll
  for (int j = 0; j < G::kDma; ++j) {
    const int s = (wq * G::kDma + j) * 64 + lane;
    const int r = s / G::kCpr, pos = s % G::kCpr;
    const int c = pos ^ (grp ? vswz<D>(r) : kswz<D>(r));
    goff[j] = r * grb + c * 16;
  }
  const unsigned my_lds =
      __builtin_amdgcn_readfirstlane(lds_addr(grp ? vbuf : kbuf) + wq * G::kDma * 1024);
  // document labels: wave 0 also copies the stage's 64 labels (16 lanes x 16
  // bytes), so it has one more copy in flight per stage than the other waves
  const int* doc_row = DOCS ? p.va.doc + static_cast<size_t>(b) * p.va.doc_stride : p.va.doc;
  const bool lab_wave = DOCS && __builtin_amdgcn_readfirstlane(wave) == 0;
  const u32x4 ldesc = make_desc(doc_row, DOCS ? static_cast<unsigned>(p.va.doc_stride) * 4u : 0u);
  const unsigned lab_lds = lds_addr(labbuf);
  // group 0 copies K(t), group 1 V(t), into ring slot `ring` (t: the
  // stage's index in ascending key order)
  auto issue_copy = [&](int t, int e, int ring) {
    const int kv0 = stage_kv0(t, e);
    const unsigned gbase = static_cast<unsigned>(kv0) * grb;
    const unsigned lbase = my_lds + ring * G::kBufBytes;
#pragma unroll
    for (int j = 0; j < G::kDma; ++j)
      copy_to_lds(desc, gbase + goff[j], __builtin_amdgcn_readfirstlane(lbase + j * 1024));
    if constexpr (DOCS) {
      if (lab_wave && lane < kBN / 4)
        copy_to_lds(ldesc, static_cast<unsigned>(kv0 + 4 * lane) * 4u,
                    __builtin_amdgcn_readfirstlane(lab_lds + ring * kBN * 4));
    }
  };
  // this wave's copies of the stage before the newest are complete
  auto wait_prev_stage = [&]() {
    if (lab_wave) wait_vm<G::kDma + 1>();
    else wait_vm<G::kDma>();
  };

  // whole lists: the first two stages (both in the first key tile) are
  // copied as soon as the list head is known; a second stage past Skv reads
  // zeros and is never used
  if (early && n_entries > 0) {
    issue_copy(0, e_head, 0);
    issue_copy(1, e_head, 1);
  }

  int e_first = 0;
  if (p.splits > 1) {
    // this split's contiguous part of the list
    const int n_all = n_entries;
    e_first = static_cast<int>(static_cast<long long>(n_all) * split / p.splits);
    n_entries = static_cast<int>(static_cast<long long>(n_all) * (split + 1) / p.splits) - e_first;
  }
  if constexpr (PK) {
    // every packed row lies in query tile 0, so a tile is visited when
    // either half admits a pair, and skips the per-element mask only when
    // both halves are full (half 1 has no rows when Sq <= 128)
    for (int i = tid; i < n_entries; i += kThreads) {
      const int e = list ? list[e_first + i] : unlisted(e_first + i);
      const bool full = (e & 2) && ((e & 8) || p.Sq <= kPairHalf);
      ents[i] = (e & ~15) | ((e & 5) ? (full ? 0xF : 0x5) : 0);
    }
  } else if (list) {
    int i = tid;
    if (early && n_head < 0) {   // the first kThreads entries are already in flight
      if (tid < n_entries) ents[tid] = e_spec;
      i += kThreads;
    }
    for (; i < n_entries; i += kThreads) ents[i] = list[e_first + i];
  } else {
    for (int i = tid; i < n_entries; i += kThreads) ents[i] = unlisted(e_first + i);
  }
  if constexpr (MOD == kModRelBias) {
    // decode mode: the tables of all rep heads of the group, one after another
    const int n_tab = 2 * p.va.rel_max + 1;
    const int h0 = PK ? kvh * rep : __builtin_amdgcn_readfirstlane(h);
    for (int j = 0; j < (PK ? rep : 1); ++j)
      stage_rel_table(p.va, h0 + j, (lds_f32*)(rtab) + j * n_tab, tid, kThreads);
  }
  __syncthreads();
  int n_stages = kSPT * n_entries;
  if (n_entries > 0) {
    // stages of the last tile that start at or past Skv are dropped
    const int last = ents[n_entries - 1] >> 4;
    const int kept = (p.Skv - last * kTile + kBN - 1) / kBN;
    n_stages -= kSPT - min(kept, kSPT);
  }
  // step u of the loop visits stage ord(u) of the ascending key order;
  // steps past the end clamp to the last stage (their copies are never issued)
  auto ord = [&](int u) -> int { return kDesc ? max(n_stages - 1 - u, 0) : min(u, max(n_stages - 1, 0)); };
  auto ent = [&](int u) -> int { return ents[ord(u) / kSPT]; };

  // ---- running state
  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  // The running max starts as -inf, hidden from the compiler: a copy of the
  // first loop step that knew it would compute the first stage's scores from
  // a constant exponent base, with other instructions (and roundings) than
  // the loop body, and which stage comes first depends on the block mask.
  float m_run = -INFINITY;
  asm("" : "+v"(m_run));
  // Kept beside it, so that a stage needs no test of m_run against -inf:
  // the exponent base (m_run, or 0 while the row has none) and the rescale
  // threshold (kRescaleLog2 above the base, or -inf while there is none).
  float base_run = 0.f, thr_run = -INFINITY;
  asm("" : "+v"(base_run), "+v"(thr_run));
  float l_run = 0.f;
  using SM = ScoreMod<MOD>;
  const int q_pos = q_row + p.va.q_offset;   // position in the key sequence
  const typename SM::Lane sml = [&] {
    typename SM::Lane L = SM::lane(p.va, h, q_pos);
    if constexpr (MOD == kModRelBias) L.tab = (lds_cf32*)(rtab) + hl * (2 * p.va.rel_max + 1) + p.va.rel_max;
    return L;
  }();
  const int doc_q = (DOCS && q_ok) ? doc_row[q_pos] : 0;
  // lanes of real rows: wave-wide softmax decisions are voted by these only
  const uint64_t qmask = __builtin_amdgcn_ballot_w64(q_ok);
  auto rows_any = [&](bool c) { return (__builtin_amdgcn_ballot_w64(c) & qmask) != 0; };

  // a wave's keys of a stage: all, or (key split) its group's 32-key half
  constexpr int KB = KS ? 1 : G::kKB, CH = KS ? 2 : G::kCH;
  constexpr int kBW = KB * 32;
  const int koff_w = KS ? 32 * grp : 0;
  bf16x8 pf[CH];

  // S^T(t) = K(t) Q^T: KB 32-key blocks, fragment reads 4 ahead of the MFMAs
  auto qk = [&](int ring, f32x16 (&s)[KB]) {
    const unsigned char* kb_ = kbuf + ring * G::kBufBytes;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_ + koff_at(c) + (kb * 32 + koff_w) * RB);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
#pragma unroll
    for (int i = 0; i < KB * DC - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);
  };

  // O^T += V(t)^T P^T(t): the A fragment of (db, ch) is two transposing reads
  // (keys 16 ch + 4 g + 0..3 and 16 ch + 8 + 4 g + 0..3, matching the key order
  // of the P^T operand built from the S^T accumulators)
  auto pv = [&](int ring) {
    const unsigned char* vb = vbuf + ring * G::kBufBytes;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const unsigned char* a0 = vb + voff_at(db) + (16 * ch + koff_w) * RB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 8 * RB));
        const i16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[ch], o[db],
                                                        0, 0, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x0100, 8, 0);
#pragma unroll
    for (int i = 0; i < CH * DB - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);
  };

  // online softmax of one stage: scores -> P^T (bf16) in pf, running max/sum
  auto softmax = [&](const f32x16 (&s)[KB], int kv0, bool full, int ring) {
    // u = t - base0: the modified scores in log2 units, measured from this
    // lane's exponent base at the start of the stage (0 while it has none);
    // each score mod folds the base into a per-stage constant
    const float base0 = base_run;
    const int dk0 = kv0 + 4 * g - q_pos;   // key kv0 + 4 g + c is at distance dk0 + c
    float t[KB * 16];
    // Relative bias: when every distance of the stage, over the wave's 32
    // rows, lies beyond the clip distance, all scores take the same end entry
    // of the table (one wave-uniform LDS read instead of one per score).
    bool clipped = false;
    float clip_add = 0.f;
    if constexpr (MOD == kModRelBias) {
      // the wave's rows lie in [qw, qw + span]: lane 0 holds the first of 32
      // consecutive rows; in decode mode any row of query tile 0
      const int qw = PK ? p.va.q_offset : __builtin_amdgcn_readfirstlane(q_pos);
      const int span = PK ? p.Sq - 1 : 31;
      const int R = p.va.rel_max;
      const bool below = kv0 + kBW - 1 - qw < -R;   // largest distance below -R
      const bool above = kv0 - (qw + span) > R;     // smallest distance above R
      clipped = below || above;
      if (clipped) clip_add = sml.tab[below ? -R : R] * kLog2e;
    }
    if (clipped) {
      const float cb = clip_add - base0;
#pragma unroll
      for (int i = 0; i < KB * 16; ++i) t[i] = __builtin_fmaf(s[i >> 4][i & 15], p.va.c1, cb);
    } else {
      const typename SM::Stage st = SM::stage(p.va, sml, dk0, base0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          t[kb * 16 + r] = SM::shifted(s[kb][r], p.va, sml, st, kb * 32 + 8 * (r >> 2) + (r & 3));
    }
    const float ninf = -INFINITY;
    if (!full) {
      // The causal part (with its prefix), the window and the key range each
      // admit an interval of key positions for this row, so together they
      // admit keys kk0 + c for c in [lo, hi], where element (kb, i, e) of this
      // lane is key kk0 + c with c = 32 kb + 8 i + e (0 <= c <= kBW - 5).
      // Bounds are formed in 64 bits and clamped to the stage.
      const bool causal = p.mask_kind & kMaskCausal;
      const bool window = p.mask_kind & kMaskWindow;
      const int kk0 = kv0 + 4 * g;
      const long long d = static_cast<long long>(q_pos) - kk0;
      long long hi = static_cast<long long>(p.Skv) - 1 - kk0;
      if (causal) hi = min(hi, max(d, static_cast<long long>(p.va.prefix) - 1 - kk0));
      const long long lo = window ? d - p.va.window + 1 : 0LL;
      int hi_c = static_cast<int>(min(max(hi, -1LL), static_cast<long long>(kBW)));
      int lo_c = static_cast<int>(min(max(lo, 0LL), static_cast<long long>(kBW)));
      // Documents: when the stage's keys all carry one label, a row's label
      // test has one answer for all of them and is folded into the interval
      // (a row of another document admits none); otherwise every element
      // compares its key's staged label with the row's.
      bool need_doc = false;
      if constexpr (DOCS) {
        const int lk = labbuf[ring * kBN + koff_w + (lane & (kBW - 1))];
        const int l0 = __builtin_amdgcn_readfirstlane(lk);
        if (wave_all(lk == l0)) {
          if (doc_q != l0) hi_c = -1;
        } else {
          need_doc = true;
        }
      }
      asm("" : "+v"(hi_c), "+v"(lo_c));   // compare the clamped 32-bit bounds
      // Each test runs only when some lane of the wave needs it (a stage on
      // the diagonal needs the upper bound alone, one on the window's far
      // edge the lower bound alone), as one compare and one select per element.
      const bool need_lo = !wave_all(lo_c <= 0);
      const bool need_hi = !wave_all(hi_c >= kBW - 1);
      if (need_doc) {
        const int* lab = labbuf + ring * kBN + koff_w + 4 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 l4 = *reinterpret_cast<const u32x4*>(lab + kb * 32 + 8 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              mask_in_place(t[kb * 16 + 4 * i + e],
                            __builtin_amdgcn_ballot_w64(static_cast<int>(l4[e]) == doc_q), ninf);
          }
      }
      if (need_lo) {
#pragma unroll
        for (int j = 0; j < KB * 16; ++j) {
          const int c = (j >> 4) * 32 + 8 * ((j >> 2) & 3) + (j & 3);
          mask_in_place(t[j], __builtin_amdgcn_ballot_w64(c >= lo_c), ninf);
        }
      }
      if (need_hi) {
#pragma unroll
        for (int j = 0; j < KB * 16; ++j) {
          const int c = (j >> 4) * 32 + 8 * ((j >> 2) & 3) + (j & 3);
          mask_in_place(t[j], __builtin_amdgcn_ballot_w64(c <= hi_c), ninf);
        }
      }
    }
    // P = exp2(t) rounded to bf16 into pf; returns this lane's fp32 sum of
    // the unrounded values
    auto exps = [&]() -> float {
      // four partial sums, so that the adds form four short chains instead
      // of one long one (-0 + x = x, so the first add of each folds away)
      float acc4[4] = {-0.f, -0.f, -0.f, -0.f};
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int kb = ch >> 1, r0 = (ch & 1) * 8;
        unsigned w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool poly = ch < FLEXATTN_EXP2_POLY_CHUNKS;
          const float x0 = t[kb * 16 + r0 + 2 * j], x1 = t[kb * 16 + r0 + 2 * j + 1];
          const float p0 = poly ? exp2_poly(x0) : __builtin_amdgcn_exp2f(x0);
          const float p1 = poly ? exp2_poly(x1) : __builtin_amdgcn_exp2f(x1);
          w[j] = pack_bf16(p0, p1);
          acc4[j] += p0 + p1;
        }
        const u32x4 wv = {w[0], w[1], w[2], w[3]};
        pf[ch] = __builtin_bit_cast(bf16x8, wv);
      }
      return (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    };
    float ls = 0.f;
    // Exponent base. Any base gives the same O / l and base + log2 l in exact
    // arithmetic; the base is raised to the row max only when some score of
    // the stage exceeds it by more than 2^kRescaleLog2 (the conditional
    // rescaling of the FA4 forward-pass fixes). With soft-capping the stage
    // is first computed against the current base and checked afterwards:
    // every weight is at most the lane's row sum, so a sum <= 2^kRescaleLog2
    // (which also rules out inf) proves no weight overflowed the bound, and
    // the max is computed only when the check fails or no base exists yet.
    // This pays off with soft-capping, whose tanh already keeps the vector
    // ALU busy; without it the denser exponential stream slows the other
    // wave's matrix products more than the skipped max saves. The other
    // variants take the max first.
    // After a failed check the base moves to the row max whenever it grew at
    // all, so that the following stages pass the check again.
    // Only rows that exist take part in these wave-wide decisions: a padding
    // row past Sq sees every key of a full tile but only the keys its mask
    // admits in a partial one, and must not make the real rows of its wave
    // rescale in one case and not in the other.
    bool need_max = true;
    bool checked = false;   // soft-capping: the stage failed the sum check
    if constexpr (MOD == kModSoftcap) {
      if (!rows_any(m_run == -INFINITY)) {
        ls = exps();
        need_max = rows_any(!(ls <= kSumLimit));
        checked = true;
      }
    }
    if (need_max) {
      // row max as four chains of three-input maxima, joined at the end
      float mx4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int i = 0; i < KB * 16; i += 8)
#pragma unroll
        for (int c = 0; c < 4; ++c) mx4[c] = fmaxf(fmaxf(mx4[c], t[i + c]), t[i + 4 + c]);
      float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
      mx = max_pair32_nn(mx);   // the row max, relative to base0
      // after a failed check every real row has a base: move it on any growth
      const float thr = checked ? 0.f : thr_run;
      if (rows_any(mx > thr)) {
        const float m_new = fmaxf(m_run, mx + base0);
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] *= alpha;
        const float shift = none ? 0.f : m_new - base0;
#pragma unroll
        for (int i = 0; i < KB * 16; ++i) t[i] -= shift;
        m_run = m_new;
        base_run = none ? 0.f : m_new;
        thr_run = none ? -INFINITY : kRescaleLog2;
      }
      ls = exps();
    }
    l_run += ls;
  };

  // Barrier between slots. Without the LDS wait of __syncthreads: the copies
  // into LDS are ordered by the explicit vmcnt waits before it, and every
  // LDS read of a slot is consumed by that slot's own instructions. The empty
  // asm statements keep the compiler from moving memory accesses across it.
  auto slot_barrier = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- prologue: stages 0 and 1 (group 0 copies K, group 1 copies V)
  const int T = n_stages;
  if (!early && T > 0) issue_copy(ord(0), ent(0), 0);
  if (!early && T > 1) issue_copy(ord(1), ent(1), 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Group 1 runs one slot behind (ping-pong), except at D = 256: its stages
  // hold 32 keys, so a wave's softmax is half as long as its matrix slot, and
  // the two waves of a SIMD do better taking the matrix cores back to back and
  // exponentiating together (A/B on one machine: 825 -> 952 TFLOPS on the causal
  // GQA workload at D = 256; 14% slower at D = 64 and 128).
  constexpr bool kInPhase = D == 256;
  if (!kInPhase && grp == 1) __syncthreads();

  int e_prev = 0, e_cur = ent(0), e_next = ent(1);
  int ring = 0;   // ring slot of stage u (u % 3); stage u - 1 and u + 2 share slot (u + 2) % 3
  const int sh = PACK == 3 ? 0 : 2 * grp;   // mode 3: every row lies in half 0
  for (int u = 0; u < T; ++u) {
    const int ring_old = ring == 0 ? kRing - 1 : ring - 1;
    const int ec = __builtin_amdgcn_readfirstlane(e_cur) >> sh;
    const int ep = __builtin_amdgcn_readfirstlane(e_prev) >> sh;
    const bool do_s = live && (ec & 1);    // this half has admitted pairs in stage u
    const bool do_pv = live && u >= 1 && (ep & 1);

    // matrix slot. S^T is computed even for a stage this half skips (a
    // conditional product would make the scores a loop phi, which the compiler
    // resolves by copying all 32 of them every stage).
    f32x16 s[KB];
    __builtin_amdgcn_s_setprio(1);   // the multiplying wave goes first on its SIMD
    if (live) qk(ring, s);
    if (do_pv) pv(ring_old);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    slot_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // vector slot
    const int e_n2 = ent(u + 2);
    if (do_s)
      softmax(s, stage_kv0(ord(u), __builtin_amdgcn_readfirstlane(e_cur)) + koff_w, ((ec >> 1) & 1) != 0, ring);
    if (u + 2 < T) {
      issue_copy(ord(u + 2), __builtin_amdgcn_readfirstlane(e_n2), ring_old);
      wait_prev_stage();   // this group's copies of stage u + 1 are complete
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_sched_barrier(0);
    slot_barrier();
    __builtin_amdgcn_sched_barrier(0);

    e_prev = e_cur;
    e_cur = e_next;
    e_next = e_n2;
    ring = ring == kRing - 1 ? 0 : ring + 1;
  }
  // last matrix slot: O^T += V^T P^T of the last stage; its vector slot is empty
  {
    const int ep = __builtin_amdgcn_readfirstlane(e_prev) >> sh;
    __builtin_amdgcn_s_setprio(1);
    if (live && T >= 1 && (ep & 1)) pv(ring == 0 ? kRing - 1 : ring - 1);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __syncthreads();
  }
  if (!kInPhase && grp == 0) __syncthreads();   // matches group 1's extra barrier

  if constexpr (KS) {
    // Merge the two key halves: each wave of group 1 hands its base, partial
    // sums and O^T to its partner in group 0 through the idle stage rings
    // (waves 0, 1 in the K ring, 2, 3 in the V ring), register by register
    // (64 lanes x 4 bytes contiguous). Each half's O and l are relative to
    // its own base m_w; those of all the keys are the sums of 2^(m_w - M) O_w
    // and 2^(m_w - M) l_w, M the larger base (a half that admitted no key
    // has m_w = -inf and weighs 0).
    constexpr int XW = (2 + 16 * DB) * 64;   // floats per wave
    static_assert(2 * XW * 4 <= kRing * G::kBufBytes, "exchange fits the stage rings");
    float* const xch = reinterpret_cast<float*>(wq < 2 ? kbuf : vbuf) + (wq & 1) * XW;
    if (live && grp == 1) {
      xch[lane] = m_run;
      xch[64 + lane] = l_run;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[(2 + 16 * db + i) * 64 + lane] = o[db][i];
    }
    __syncthreads();
    if (live && grp == 0) {
      const float m1 = xch[lane], l1 = xch[64 + lane];
      const float mm = fmaxf(m_run, m1);
      const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      l_run = a0 * l_run + a1 * l1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = a0 * o[db][i] + a1 * xch[(2 + 16 * db + i) * 64 + lane];
      m_run = mm;
    }
    __syncthreads();   // the exchange is read before the epilogue reuses the rings
  }
  // rows this wave writes (key split: group 0's copy of the rows)
  const bool out_ok = q_ok && (!KS || grp == 0);

  // ---- epilogue: normalise, LSE, store
  const float l_tot = sum_pair32(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (p.splits > 1) {
    // this split's normalised rows and LSE, merged by attn_decode_merge_kernel;
    // workspace rows [split][b][h][q_row] (in decode mode h = kvh rep + hl)
    if (out_ok) {
      const size_t wrow = ((static_cast<size_t>(split) * p.B + b) * p.H + h) * p.Sq + q_row;
      float* const wo = p.ws_o + wrow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + 8 * i + 4 * g;
          const f32x4 vv = {o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                            o[db][4 * i + 3] * inv};
          *reinterpret_cast<f32x4*>(wo + d0) = vv;
        }
      if (g == 0) p.ws_lse[wrow] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
    }
  } else if constexpr (!PK) {
    // O through LDS: each wave writes its 32 rows row-major into the idle
    // stage buffers (16-byte chunks XOR-permuted by row, so neither side has
    // bank conflicts) and stores whole rows, 16 bytes per lane. A store then
    // covers 64 / CPP complete rows, where a direct store from the O^T
    // fragments would put 16 bytes into each of 32 rows.
    constexpr int DP = D < 128 ? D : 128;   // d values staged per pass
    constexpr int CPP = DP / 8;             // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPP;           // rows per store instruction
    static_assert(4 * 32 * DP * 2 <= kRing * G::kBufBytes, "output staging fits a stage ring");
    unsigned char* const stg = (grp ? vbuf : kbuf) + wq * 32 * DP * 2;
    __bf16* const obase = static_cast<__bf16*>(p.out) + b * p.o_sb + h * p.o_sh;
    const int row0 = q_row - l32;   // first query row of the wave
#pragma unroll
    for (int ps = 0; ps < D / DP; ++ps) {
#pragma unroll
      for (int db = ps * DP / 32; db < (ps + 1) * DP / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = (db * 32 - ps * DP) / 8 + i;   // chunk of d = 32 db + 8 i + 4 g
          const u32x2 vv = {pack_bf16(o[db][4 * i] * inv, o[db][4 * i + 1] * inv),
                            pack_bf16(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv)};
          *reinterpret_cast<u32x2*>(stg + l32 * DP * 2 + ((c ^ (l32 % CPP)) * 16) + g * 8) = vv;
        }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 32 / RPI; ++j) {
        const int r = j * RPI + lane / CPP, c = lane % CPP;
        const u32x4 w = *reinterpret_cast<const u32x4*>(stg + r * DP * 2 + ((c ^ (r % CPP)) * 16));
        if (row0 + r < p.Sq && (!KS || grp == 0))
          *reinterpret_cast<u32x4*>(obase + static_cast<size_t>(row0 + r) * p.o_sr + ps * DP + c * 8) = w;
      }
      if (ps + 1 < D / DP) __syncthreads();   // read back before the next pass overwrites
    }
    if (p.lse && g == 0 && out_ok)
      p.lse[q_head + q_row] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  } else if (out_ok) {
    __bf16* const obase = static_cast<__bf16*>(p.out) + b * p.o_sb + h * p.o_sh;
    const size_t orow = static_cast<size_t>(q_row) * p.o_sr;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        const u32x2 vv = {pack_bf16(o[db][4 * i] * inv, o[db][4 * i + 1] * inv),
                          pack_bf16(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv)};
        *reinterpret_cast<u32x2*>(obase + orow + d0) = vv;
      }
    if (p.lse && g == 0)
      p.lse[q_head + q_row] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int MOD, bool DOCS, int PACK>
hipError_t launch_t(const FwdLaunch& p, hipStream_t stream) {
  const int np = (p.Sq + kBM - 1) / kBM;
  const long long total = ((PACK == 1 || PACK == 2) ? static_cast<long long>(p.B) * p.Hkv
                                : static_cast<long long>(p.B) * p.H * np) * p.splits;
  const long long per = (total + kXcds - 1) / kXcds;
  note_launch("attn_fwd_pp_kernel<%d, %d, %s, %d> grid %lld x %d splits %d", D, MOD, DOCS ? "true" : "false",
              PACK, per * kXcds, kThreads, p.splits);
  hipLaunchKernelGGL((attn_fwd_pp_kernel<D, MOD, DOCS, PACK>), dim3(static_cast<unsigned>(per * kXcds)),
                     dim3(kThreads), 0, stream, p, p.kv_count, p.kv_list);
  return hipGetLastError();
}

template <int D, bool DOCS, int PACK>
hipError_t launch_mod(const FwdLaunch& p, hipStream_t stream) {
  switch (p.mod_kind) {
    case kModNone: return launch_t<D, kModNone, DOCS, PACK>(p, stream);
    case kModAlibi: return launch_t<D, kModAlibi, DOCS, PACK>(p, stream);
    case kModSoftcap: return launch_t<D, kModSoftcap, DOCS, PACK>(p, stream);
    case kModRelBias: return launch_t<D, kModRelBias, DOCS, PACK>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int PACK>
hipError_t launch_dims(const FwdLaunch& p, hipStream_t stream) {
  if (p.splits < 1) return hipErrorInvalidValue;
  const bool docs = p.mask_kind & kMaskDocument;
  if (p.D == 256) {
    if constexpr (PACK >= 2) return hipErrorInvalidValue;
    else return docs ? launch_mod<256, true, PACK>(p, stream) : launch_mod<256, false, PACK>(p, stream);
  }
  if (p.D == 128) return docs ? launch_mod<128, true, PACK>(p, stream) : launch_mod<128, false, PACK>(p, stream);
  if (p.D == 64) return docs ? launch_mod<64, true, PACK>(p, stream) : launch_mod<64, false, PACK>(p, stream);
  return hipErrorInvalidValue;
}

// Merge of the decode splits: for every (b, head, row) the split results
// (O_s normalised, LSE_s) combine as LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s (a row no split admitted anything for keeps
// O = 0, LSE = -inf). One thread per 4 values of d.
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(FwdLaunch p) {
  const int rep = p.H / p.Hkv, rows = rep * p.Sq, dq = p.D / 4;
  const long long n = static_cast<long long>(p.B) * p.Hkv * rows * dq;
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n) return;
  const int d0 = static_cast<int>(t % dq) * 4;
  const long long grow = t / dq;   // (b, kvh, r)
  const int r = static_cast<int>(grow % rows);
  const long long bk = grow / rows;
  const int kvh = static_cast<int>(bk % p.Hkv), b = static_cast<int>(bk / p.Hkv);
  const size_t split_rows = static_cast<size_t>(p.B) * p.Hkv * rows;
  float mx = -INFINITY;
  for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.ws_lse[s * split_rows + grow]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (mx > -INFINITY) {
    for (int s = 0; s < p.splits; ++s) {
      const float w = __expf(p.ws_lse[s * split_rows + grow] - mx);
      tot += w;
      acc += w * *reinterpret_cast<const f32x4*>(p.ws_o + (s * split_rows + grow) * p.D + d0);
    }
    acc *= 1.0f / tot;
  }
  const int hl = r / p.Sq, q_row = r - hl * p.Sq, h = kvh * rep + hl;
  __bf16* const orow = static_cast<__bf16*>(p.out) + b * p.o_sb + h * p.o_sh + static_cast<size_t>(q_row) * p.o_sr;
  const u32x2 vv = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
  *reinterpret_cast<u32x2*>(orow + d0) = vv;
  if (p.lse && d0 == 0)
    p.lse[(static_cast<size_t>(b) * p.H + h) * p.Sq + q_row] = mx > -INFINITY ? mx + __logf(tot) : -INFINITY;
}

// Split results of flexattn_decode_static, whose callers cannot allocate
// device memory: a file-scope array, one copy per device, held until the
// process ends. Host code never names it as an address (in host code the name
// stands for a host-side shadow, not device memory); it uses the address that
// hipGetSymbolAddress returns for the current device.
__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t static_scratch(int device, void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    // once per device, with that device current (the caller's check)
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[device] = a;
  }
  *ptr = addr[device];
  return hipSuccess;
}

// Sq <= 128 (every row in the first half of the one query tile) and D <= 128
// take the key split
hipError_t launch_attn_fwd_pp(const FwdLaunch& p, hipStream_t stream) {
  return p.Sq <= kPairHalf && p.D <= 128 ? launch_dims<3>(p, stream) : launch_dims<0>(p, stream);
}

// Split-KV: a group's rows packed into one workgroup when they fit (decode
// mode; with at most 128 rows and D <= 128, the key halves of every stage
// split between the two groups), else the regular mapping with every query
// tile's list split.
hipError_t launch_attn_decode(const FwdLaunch& p, hipStream_t stream) {
  const long long packed_rows = static_cast<long long>(p.H / p.Hkv) * p.Sq;
  hipError_t e = packed_rows <= kPairHalf && p.D <= 128 ? launch_dims<2>(p, stream)
                 : packed_rows <= kBM            ? launch_dims<1>(p, stream)
                                                 : launch_attn_fwd_pp(p, stream);
  if (e != hipSuccess || p.splits <= 1) return e;
  const long long n = static_cast<long long>(p.B) * p.Hkv * (p.H / p.Hkv) * p.Sq * (p.D / 4);
  note_launch("attn_decode_merge_kernel grid %lld x 256", (n + 255) / 256);
  hipLaunchKernelGGL(attn_decode_merge_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace fa
