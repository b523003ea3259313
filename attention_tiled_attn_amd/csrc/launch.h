// launch.h - internal interface between the C ABI (api.cpp) and the HIP kernels.
// Every launch function assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "variant_args.h"

namespace fa {

// Block-mask lists are kept per 256-row query tile, made of two 128-row
// halves; entries are (kv_tile << 4) | full1 << 3 | any1 << 2 | full0 << 1 | any0.
constexpr int kPairHalf = 128;
// Largest key-tile count whose list the bf16 kernel caches in LDS.
constexpr int kPairMaxKeyTiles = 2048;

struct FwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;          // may be null
  int B, H, Hkv, Sq, Skv, D;
  int is_fp32;         // element type of q/k/v/out
  int mask_kind;
  int mod_kind;
  VariantArgs va;
  // element strides of q, k, v, out: batch and head (64-bit) and row
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_sr, k_sr, v_sr, o_sr;
  // block mask (kv_count == nullptr: visit every key tile as partial);
  // nq counts 256-row query tiles
  const int* kv_count;
  const int* kv_list;
  int nq, nk, bm_num_b;
  // key-tile lists split over `splits` >= 1 workgroups (launch_attn_decode;
  // 1 for launch_attn_fwd). When rep * Sq <= 256 the H/Hkv query heads of a
  // key/value head share a workgroup as packed rows (decode mode). With
  // splits > 1 each writes its rows' normalised O (float32) and LSE to
  // ws_o [splits][B][H][Sq][D] and ws_lse [splits][B][H][Sq], merged by a
  // second kernel
  int splits;
  float* ws_o;
  float* ws_lse;
};

hipError_t launch_attn_fwd(const FwdLaunch& p, hipStream_t stream);
hipError_t launch_attn_decode(const FwdLaunch& p, hipStream_t stream);

// Static scratch of flexattn_decode_static (bytes; the header's
// FLEXATTN_STATIC_SCRATCH_BYTES), and its device address on `device`, which
// must be the current device. Looked up once per device, then cached.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(int device, void** ptr);
// bf16 inputs with nk <= kPairMaxKeyTiles (256-row ping-pong kernel)
hipError_t launch_attn_fwd_pp(const FwdLaunch& p, hipStream_t stream);

struct BwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int B, H, Hkv, Sq, Skv, D;
  int mask_kind;
  int mod_kind;
  float scale;
  VariantArgs va;
  const int* kv_count;   // block mask (256-row query tiles), or nullptr
  const int* kv_list;
  int nq, nk, bm_num_b;
  // element strides {batch, head} and row strides: q and dq share q's, k and
  // dk k's, v and dv v's, out and dout out's (LSE and delta are contiguous)
  long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_sr, k_sr, v_sr, o_sr;
};

// dQ (and delta) first, then dK/dV, both on `stream`
hipError_t launch_attn_bwd(const BwdLaunch& p, hipStream_t stream);

struct MaskLaunch {
  int mask_kind;
  int window;
  const int* doc;
  int doc_stride;
  int q_offset;   // position of query row 0
  int prefix;     // prefix-LM boundary (0 = none)
  int B, Sq, Skv;
  int nq, nk, num_b;
  int* kv_count;
  int* kv_list;
};

hipError_t launch_block_mask(const MaskLaunch& p, hipStream_t stream);

// Dispatch log (FLEXATTN_LOG): the launch functions note each kernel they
// launch (name, template arguments, grid), printf-style; the entry point
// prints the notes of its call when it returns. No-op when the log is off.
__attribute__((format(printf, 1, 2))) void note_launch(const char* fmt, ...);

}  // namespace fa
