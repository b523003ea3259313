// api.cpp - the C ABI declared in include/flexattn.h: argument validation
// (pure host code, done before any HIP call), dispatch, error reporting.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <string>

#include "../../include/flexattn.h"
#include "launch.h"

static_assert(fa::kStaticScratchBytes == FLEXATTN_STATIC_SCRATCH_BYTES, "static scratch size");

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* where) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e),
                static_cast<int>(e));
  return FLEXATTN_ERR_HIP;
}

// ---- dispatch log. FLEXATTN_LOG set to anything but "" or "0" makes every
// entry point that can launch work print one line on stderr when it returns:
// its arguments, each kernel it launched (template arguments, grid and
// workgroup size) and its status. Read once per process; when off, a call
// pays one test of a cached flag.
bool log_enabled() {
  static const bool on = [] {
    const char* s = std::getenv("FLEXATTN_LOG");
    return s && *s && std::strcmp(s, "0") != 0;
  }();
  return on;
}

thread_local std::string g_launches;   // kernels noted by the current call

void log_begin() {
  if (log_enabled()) g_launches.clear();
}

const char* dtype_name(const flexattn_params* prm) {
  if (!prm) return "bf16";
  return prm->dtype == FLEXATTN_BF16 ? "bf16" : prm->dtype == FLEXATTN_FP32 ? "fp32" : "?";
}

__attribute__((format(printf, 3, 4))) void log_end(const char* entry, int status, const char* fmt, ...) {
  if (!log_enabled()) return;
  char args[384];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(args, sizeof(args), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[flexattn] %s(%s) -> %s -> %d (%s)\n", entry, args,
               g_launches.empty() ? "no launch" : g_launches.c_str(), status, flexattn_strerror(status));
  g_launches.clear();
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

const flexattn_params kDefaultParams = {FLEXATTN_BF16, 0, 0.f, nullptr, nullptr, 0, 0, 0, nullptr, 0,
                                        {0, 0, 0}, {0, 0, 0}, {0, 0, 0}, {0, 0, 0}};

// Effective strides {batch, head, row} of one tensor: the given ones, or the
// contiguous layout [heads][rows][D] per batch when all three are zero.
struct Strides {
  long long b, h, r;
};
Strides strides_of(const long long (&s)[3], int heads, int rows, int D) {
  if (s[0] == 0 && s[1] == 0 && s[2] == 0)
    return {static_cast<long long>(heads) * rows * D, static_cast<long long>(rows) * D, D};
  return {s[0], s[1], s[2]};
}
// Checks of one tensor's layout: element strides, 16-byte alignment of every
// row, and 32-bit byte offsets within one (batch, head) slice including one
// query tile of rows past the end, which the kernels read as zeros.
int check_layout(const Strides& s, int rows, int D, long long esz) {
  if (s.b < 0 || s.h < 0 || s.r < D) return FLEXATTN_ERR_ARG;
  const long long q16 = 16 / esz;
  if (s.b % q16 || s.h % q16 || s.r % q16) return FLEXATTN_ERR_ALIGN;
  if ((static_cast<long long>(rows) + FLEXATTN_QTILE) * s.r * esz > INT_MAX) return FLEXATTN_ERR_OVERFLOW;
  return FLEXATTN_OK;
}

// True when distinct elements [n][heads][rows][D] of a layout never share an
// address. Sufficient test: ordered by stride, every dimension of extent > 1
// steps over the whole span of the dimensions below it. The backward writes
// its gradients with the strides of q, k and v, so a broadcast (stride 0) or
// otherwise overlapping input would make several workgroups write one element.
bool non_overlapping(const Strides& s, int n, int heads, int rows, int D) {
  struct Dim { long long stride, extent; };
  Dim d[4] = {{1, D}, {s.r, rows}, {s.h, heads}, {s.b, n}};
  std::sort(d, d + 4, [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
  long long span = 1;   // elements covered by the dimensions taken so far
  for (const Dim& x : d) {
    if (x.extent <= 1) continue;
    if (x.stride < span) return false;
    span = x.stride * x.extent;
  }
  return true;
}

constexpr int kMaskBits = FLEXATTN_MASK_CAUSAL | FLEXATTN_MASK_WINDOW | FLEXATTN_MASK_DOCUMENT |
                          FLEXATTN_MASK_PREFIX;

// The mask parameters a block mask depends on: 0 where the kind does not use
// them (q_offset is used by every positional mask).
struct MaskKey {
  int window, q_offset, prefix;
};
MaskKey mask_key(int mask_kind, const flexattn_params* prm) {
  MaskKey m{0, 0, 0};
  if (mask_kind & FLEXATTN_MASK_WINDOW) m.window = prm->window;
  if (mask_kind & FLEXATTN_MASK_PREFIX) m.prefix = prm->prefix;
  if (mask_kind != FLEXATTN_MASK_NONE) m.q_offset = prm->q_offset;
  return m;
}

// Checks shared by the forward pass and the block-mask builder.
int check_mask_args(int mask_kind, const flexattn_params* prm, int B, int Sq, int Skv) {
  if (B < 1 || Sq < 1 || Skv < 1) return FLEXATTN_ERR_SHAPE;
  if (mask_kind < 0 || (mask_kind & ~kMaskBits)) return FLEXATTN_ERR_UNSUPPORTED;
  if ((mask_kind & FLEXATTN_MASK_WINDOW) && prm->window < 1) return FLEXATTN_ERR_ARG;
  if (mask_kind & FLEXATTN_MASK_PREFIX) {
    if (!(mask_kind & FLEXATTN_MASK_CAUSAL) || prm->prefix < 0) return FLEXATTN_ERR_ARG;
  }
  if (prm->q_offset < 0) return FLEXATTN_ERR_ARG;
  // query positions i + q_offset (plus one query tile of rows past the end)
  // stay in int range
  if (static_cast<long long>(Sq) + prm->q_offset + FLEXATTN_QTILE > INT_MAX) return FLEXATTN_ERR_OVERFLOW;
  if (mask_kind & FLEXATTN_MASK_DOCUMENT) {
    if (!prm->doc_ids) return FLEXATTN_ERR_NULLPTR;
    if (!aligned(prm->doc_ids, 4)) return FLEXATTN_ERR_ALIGN;
    const long long need = std::max(static_cast<long long>(Sq) + prm->q_offset, static_cast<long long>(Skv));
    if (prm->doc_stride < need) return FLEXATTN_ERR_ARG;
    if (static_cast<long long>(B) * prm->doc_stride > INT_MAX) return FLEXATTN_ERR_OVERFLOW;
    // the kernels read a batch row's labels through a buffer descriptor with
    // 32-bit byte offsets (position * 4)
    if (prm->doc_stride > INT_MAX / 4) return FLEXATTN_ERR_OVERFLOW;
  }
  return FLEXATTN_OK;
}

}  // namespace

namespace fa {

void note_launch(const char* fmt, ...) {
  if (!log_enabled()) return;
  char line[192];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(line, sizeof(line), fmt, ap);
  va_end(ap);
  if (!g_launches.empty()) g_launches += "; ";
  g_launches += line;
}

}  // namespace fa

extern "C" {

int flexattn_version(void) { return FLEXATTN_VERSION; }

const char* flexattn_strerror(int status) {
  switch (status) {
    case FLEXATTN_OK: return "success";
    case FLEXATTN_ERR_NULLPTR: return "a required pointer is NULL";
    case FLEXATTN_ERR_SHAPE: return "invalid shape (sizes must be >= 1 and H a multiple of Hkv)";
    case FLEXATTN_ERR_UNSUPPORTED: return "unsupported head dim, dtype, mask kind or mod kind";
    case FLEXATTN_ERR_ALIGN: return "misaligned pointer (Q/K/V/O need 16 bytes, LSE and params 4)";
    case FLEXATTN_ERR_BLOCKMASK: return "block mask does not match this call";
    case FLEXATTN_ERR_OVERFLOW: return "sizes exceed the 32-bit index range";
    case FLEXATTN_ERR_HIP: return "HIP runtime error";
    case FLEXATTN_ERR_ARG: return "invalid scalar argument";
    case FLEXATTN_ERR_SCRATCH: return "the call needs more scratch than the static buffer holds";
    default: return "unknown status";
  }
}

const char* flexattn_last_error(void) { return g_last_error; }

size_t flexattn_block_mask_bytes(int B, int Sq, int Skv, int mask_kind) {
  if (B < 1 || Sq < 1 || Skv < 1 || mask_kind < 0 || (mask_kind & ~kMaskBits)) return 0;
  const size_t nb = (mask_kind & FLEXATTN_MASK_DOCUMENT) ? static_cast<size_t>(B) : 1;
  const size_t nq = static_cast<size_t>(ceil_div(Sq, FLEXATTN_QTILE));
  const size_t nk = static_cast<size_t>(ceil_div(Skv, FLEXATTN_TILE));
  return nb * nq * (1 + nk) * sizeof(int);
}

static int build_block_mask_body(int mask_kind, const flexattn_params* params, int B, int Sq, int Skv,
                                 void* buf, size_t bytes, flexattn_block_mask* out, void* stream) {
  const flexattn_params* prm = params ? params : &kDefaultParams;
  if (!buf || !out) return FLEXATTN_ERR_NULLPTR;
  int st = check_mask_args(mask_kind, prm, B, Sq, Skv);
  if (st) return st;
  if (!aligned(buf, 4)) return FLEXATTN_ERR_ALIGN;
  const size_t need = flexattn_block_mask_bytes(B, Sq, Skv, mask_kind);
  if (need == 0 || bytes < need) return FLEXATTN_ERR_ARG;
  const int nb = (mask_kind & FLEXATTN_MASK_DOCUMENT) ? B : 1;
  if (static_cast<long long>(Sq) + FLEXATTN_QTILE > INT_MAX || static_cast<long long>(Skv) + FLEXATTN_TILE > INT_MAX)
    return FLEXATTN_ERR_OVERFLOW;
  const int nq = ceil_div(Sq, FLEXATTN_QTILE), nk = ceil_div(Skv, FLEXATTN_TILE);
  if (static_cast<long long>(nb) * nq * (1LL + nk) > INT_MAX) return FLEXATTN_ERR_OVERFLOW;

  int* counts = static_cast<int*>(buf);
  int* lists = counts + static_cast<size_t>(nb) * nq;
  fa::MaskLaunch ml{};
  ml.mask_kind = mask_kind;
  ml.window = prm->window;
  ml.doc = prm->doc_ids;
  ml.doc_stride = prm->doc_stride;
  const MaskKey key = mask_key(mask_kind, prm);
  ml.q_offset = key.q_offset;
  ml.prefix = key.prefix;
  ml.B = B;
  ml.Sq = Sq;
  ml.Skv = Skv;
  ml.nq = nq;
  ml.nk = nk;
  ml.num_b = nb;
  ml.kv_count = counts;
  ml.kv_list = lists;
  hipError_t e = fa::launch_block_mask(ml, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block-mask launch");

  out->tile_q = FLEXATTN_QTILE;
  out->tile_k = FLEXATTN_TILE;
  out->nq = nq;
  out->nk = nk;
  out->num_b = nb;
  out->mask_kind = mask_kind;
  out->Sq = Sq;
  out->Skv = Skv;
  out->kv_count = counts;
  out->kv_list = lists;
  out->window = key.window;
  out->q_offset = key.q_offset;
  out->prefix = key.prefix;
  return FLEXATTN_OK;
}

int flexattn_build_block_mask(int mask_kind, const flexattn_params* params, int B, int Sq, int Skv,
                              void* buf, size_t bytes, flexattn_block_mask* out, void* stream) {
  log_begin();
  const int st = build_block_mask_body(mask_kind, params, B, Sq, Skv, buf, bytes, out, stream);
  log_end("flexattn_build_block_mask", st, "mask=0x%x B=%d Sq=%d Skv=%d bytes=%zu stream=%p", mask_kind, B, Sq,
          Skv, bytes, stream);
  return st;
}

}  // extern "C"

namespace {

// Checks shared by the forward and backward calls (everything but the
// pointers specific to each).
int check_attn_args(const flexattn_params* prm, int B, int H, int Hkv, int Sq, int Skv, int D,
                    float scale, int mask_kind, int mod_kind, const flexattn_block_mask* block_mask) {
  if (H < 1 || Hkv < 1 || H % Hkv != 0) return FLEXATTN_ERR_SHAPE;
  int st = check_mask_args(mask_kind, prm, B, Sq, Skv);
  if (st) return st;
  if (D != 64 && D != 128 && D != 256) return FLEXATTN_ERR_UNSUPPORTED;
  if (prm->dtype != FLEXATTN_BF16 && prm->dtype != FLEXATTN_FP32) return FLEXATTN_ERR_UNSUPPORTED;
  if (mod_kind < FLEXATTN_MOD_NONE || mod_kind > FLEXATTN_MOD_RELBIAS) return FLEXATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FLEXATTN_ERR_ARG;
  if (mod_kind == FLEXATTN_MOD_ALIBI) {
    if (!prm->alibi_slopes) return FLEXATTN_ERR_NULLPTR;
    if (!aligned(prm->alibi_slopes, 4)) return FLEXATTN_ERR_ALIGN;
  }
  if (mod_kind == FLEXATTN_MOD_SOFTCAP && !(prm->softcap > 0.f && std::isfinite(prm->softcap)))
    return FLEXATTN_ERR_ARG;
  if (mod_kind == FLEXATTN_MOD_RELBIAS) {
    if (!prm->rel_bias) return FLEXATTN_ERR_NULLPTR;
    if (!aligned(prm->rel_bias, 16)) return FLEXATTN_ERR_ALIGN;
    if (prm->rel_max < 0 || prm->rel_max > FLEXATTN_REL_MAX) return FLEXATTN_ERR_ARG;
  }
  // 32-bit limits: in-kernel position arithmetic is int; tensor offsets are size_t.
  const long long nq = ceil_div(Sq, FLEXATTN_QTILE);
  const long long nk = ceil_div(Skv, FLEXATTN_TILE);
  if (static_cast<long long>(Sq) + FLEXATTN_QTILE > INT_MAX || static_cast<long long>(Skv) + FLEXATTN_TILE > INT_MAX)
    return FLEXATTN_ERR_OVERFLOW;
  if (static_cast<long long>(B) * H * ceil_div(Sq, FLEXATTN_TILE) + 8 > INT_MAX) return FLEXATTN_ERR_OVERFLOW;
  if (static_cast<long long>(B) * Hkv * nk + 8 > INT_MAX) return FLEXATTN_ERR_OVERFLOW;
  // one (batch, head) slice is addressed with 32-bit byte offsets (rows up to
  // one query tile past the end are read, as zeros)
  const long long esz = prm->dtype == FLEXATTN_FP32 ? 4 : 2;
  if ((static_cast<long long>(Sq > Skv ? Sq : Skv) + FLEXATTN_QTILE) * D * esz > INT_MAX)
    return FLEXATTN_ERR_OVERFLOW;
  if (block_mask) {
    const flexattn_block_mask* bm = block_mask;
    if (bm->tile_q != FLEXATTN_QTILE || bm->tile_k != FLEXATTN_TILE || bm->nq != nq || bm->nk != nk ||
        bm->mask_kind != mask_kind || bm->Sq != Sq || bm->Skv != Skv)
      return FLEXATTN_ERR_BLOCKMASK;
    const int want_b = (mask_kind & FLEXATTN_MASK_DOCUMENT) ? B : 1;
    if (bm->num_b != want_b) return FLEXATTN_ERR_BLOCKMASK;
    const MaskKey key = mask_key(mask_kind, prm);
    if (bm->window != key.window || bm->q_offset != key.q_offset || bm->prefix != key.prefix)
      return FLEXATTN_ERR_BLOCKMASK;
    if (!bm->kv_count || !bm->kv_list) return FLEXATTN_ERR_BLOCKMASK;
  }
  return FLEXATTN_OK;
}

void fill_variant(fa::VariantArgs& va, const flexattn_params* prm, float scale, int mask_kind,
                  int mod_kind) {
  va.c1 = scale * fa::kLog2e;
  const float cap = mod_kind == FLEXATTN_MOD_SOFTCAP ? prm->softcap : 1.f;
  va.sc_in = 2.f * fa::kLog2e * scale / cap;
  va.sc_out = cap * fa::kLog2e;
  va.window = prm->window;
  va.slopes = prm->alibi_slopes;
  va.doc = prm->doc_ids;
  va.doc_stride = prm->doc_stride;
  va.q_offset = prm->q_offset;
  va.rel_bias = mod_kind == FLEXATTN_MOD_RELBIAS ? prm->rel_bias : nullptr;
  va.rel_max = mod_kind == FLEXATTN_MOD_RELBIAS ? prm->rel_max : 0;
  va.prefix = (mask_kind & FLEXATTN_MASK_PREFIX) ? prm->prefix : 0;
}

}  // namespace

extern "C" {

static int fwd_body(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                    int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                    const flexattn_params* params, const flexattn_block_mask* block_mask,
                    void* stream) {
  const flexattn_params* prm = params ? params : &kDefaultParams;
  if (!q || !k || !v || !out) return FLEXATTN_ERR_NULLPTR;
  int st = check_attn_args(prm, B, H, Hkv, Sq, Skv, D, scale, mask_kind, mod_kind, block_mask);
  if (st) return st;
  // D = 256 runs on the bf16 ping-pong kernel only
  if (D == 256 && (prm->dtype != FLEXATTN_BF16 || ceil_div(Skv, FLEXATTN_TILE) > fa::kPairMaxKeyTiles))
    return FLEXATTN_ERR_UNSUPPORTED;

  fa::FwdLaunch p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Skv = Skv;
  p.D = D;
  p.is_fp32 = prm->dtype == FLEXATTN_FP32;
  p.mask_kind = mask_kind;
  p.mod_kind = mod_kind;
  fill_variant(p.va, prm, scale, mask_kind, mod_kind);
  {
    const long long esz = p.is_fp32 ? 4 : 2;
    const Strides qs = strides_of(prm->q_stride, H, Sq, D), ks = strides_of(prm->k_stride, Hkv, Skv, D);
    const Strides vs = strides_of(prm->v_stride, Hkv, Skv, D), os = strides_of(prm->o_stride, H, Sq, D);
    int ls = check_layout(qs, Sq, D, esz);
    if (!ls) ls = check_layout(ks, Skv, D, esz);
    if (!ls) ls = check_layout(vs, Skv, D, esz);
    if (!ls) ls = check_layout(os, Sq, D, esz);
    if (ls) return ls;
    if (!non_overlapping(os, B, H, Sq, D)) return FLEXATTN_ERR_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FLEXATTN_ERR_ALIGN;
    if (lse && !aligned(lse, 4)) return FLEXATTN_ERR_ALIGN;
    p.q_sb = qs.b; p.q_sh = qs.h; p.q_sr = static_cast<int>(qs.r);
    p.k_sb = ks.b; p.k_sh = ks.h; p.k_sr = static_cast<int>(ks.r);
    p.v_sb = vs.b; p.v_sh = vs.h; p.v_sr = static_cast<int>(vs.r);
    p.o_sb = os.b; p.o_sh = os.h; p.o_sr = static_cast<int>(os.r);
  }
  p.kv_count = block_mask ? block_mask->kv_count : nullptr;
  p.kv_list = block_mask ? block_mask->kv_list : nullptr;
  p.nq = ceil_div(Sq, FLEXATTN_QTILE);
  p.nk = ceil_div(Skv, FLEXATTN_TILE);
  p.bm_num_b = block_mask ? block_mask->num_b : 1;
  p.splits = 1;   // whole key lists, output written directly
  hipError_t e = fa::launch_attn_fwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return FLEXATTN_OK;
}

int flexattn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                 int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                 const flexattn_params* params, const flexattn_block_mask* block_mask,
                 void* stream) {
  log_begin();
  const int st = fwd_body(q, k, v, out, lse, B, H, Hkv, Sq, Skv, D, scale, mask_kind, mod_kind, params,
                          block_mask, stream);
  log_end("flexattn_fwd", st, "B=%d H=%d Hkv=%d Sq=%d Skv=%d D=%d %s scale=%g mask=0x%x mod=%d block_mask=%s lse=%s stream=%p",
          B, H, Hkv, Sq, Skv, D, dtype_name(params), scale, mask_kind, mod_kind, block_mask ? "given" : "none",
          lse ? "yes" : "no", stream);
  return st;
}

size_t flexattn_decode_workspace_bytes(int B, int H, int Hkv, int Sq, int D, int splits) {
  if (B < 1 || H < 1 || Hkv < 1 || H % Hkv || Sq < 1 || (D != 64 && D != 128 && D != 256) || splits < 1 ||
      splits > 64)
    return 0;
  if (splits == 1) return 0;
  const size_t rows = static_cast<size_t>(B) * H * Sq;   // = B * Hkv * (rep * Sq)
  return static_cast<size_t>(splits) * rows * (static_cast<size_t>(D) + 1) * sizeof(float);
}

int flexattn_decode_splits(int B, int Hkv, int Skv) {
  if (B < 1 || Hkv < 1 || Skv < 1) return 1;
  const long long tiles = ceil_div(Skv, FLEXATTN_TILE);
  const long long groups = static_cast<long long>(B) * Hkv;
  const long long cap = std::max<long long>(1, std::min<long long>(tiles / 4, 64));
  // A workgroup takes ~(2 tiles / s + 3) stage times (two 64-key stages per
  // tile, ~3 stages of start and drain), and ceil(groups * s / 256) rounds
  // of workgroups run one after another: minimise their product, the
  // smallest s among equals.
  auto cost = [&](long long s) {
    return static_cast<double>((groups * s + 255) / 256) * (2.0 * static_cast<double>(tiles) / s + 3.0);
  };
  long long best = 1;
  for (long long s = 2; s <= cap; ++s)
    if (cost(s) < cost(best)) best = s;
  return static_cast<int>(best);
}

int flexattn_split_count(int B, int H, int Hkv, int Sq, int Skv) {
  if (B < 1 || H < 1 || Hkv < 1 || H % Hkv || Sq < 1 || Skv < 1) return 1;
  if (static_cast<long long>(H / Hkv) * Sq <= FLEXATTN_QTILE) return flexattn_decode_splits(B, Hkv, Skv);
  const long long items = static_cast<long long>(B) * H * ceil_div(Sq, FLEXATTN_QTILE);
  if (items >= 2 * 256) return 1;   // already about two workgroups per CU
  const long long tiles = ceil_div(Skv, FLEXATTN_TILE);
  long long s = (2 * 256 + items - 1) / items;
  s = std::min<long long>(s, std::max<long long>(1, tiles / 8));   // >= 8 key tiles per split of a full list
  return static_cast<int>(std::max<long long>(1, std::min<long long>(s, 64)));
}

}  // extern "C"

namespace {

// flexattn_decode (workspace from the caller) and flexattn_decode_static
// (use_static: the library's static scratch; workspace ignored).
int decode_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Hkv,
                int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind, const flexattn_params* params,
                const flexattn_block_mask* block_mask, int splits, void* workspace, size_t workspace_bytes,
                bool use_static, void* stream) {
  const flexattn_params* prm = params ? params : &kDefaultParams;
  if (!q || !k || !v || !out) return FLEXATTN_ERR_NULLPTR;
  int st = check_attn_args(prm, B, H, Hkv, Sq, Skv, D, scale, mask_kind, mod_kind, block_mask);
  if (st) return st;
  if (prm->dtype != FLEXATTN_BF16) return FLEXATTN_ERR_UNSUPPORTED;
  const int rep = H / Hkv;
  // packed: the rows of a group's rep query heads fit one workgroup
  const bool packed = static_cast<long long>(rep) * Sq <= FLEXATTN_QTILE;
  if (ceil_div(Skv, FLEXATTN_TILE) > fa::kPairMaxKeyTiles) return FLEXATTN_ERR_UNSUPPORTED;
  if (packed && mod_kind == FLEXATTN_MOD_RELBIAS &&
      static_cast<long long>(rep) * (2LL * prm->rel_max + 1) > fa::kRelCap)
    return FLEXATTN_ERR_UNSUPPORTED;
  if (splits < 1 || splits > 64) return FLEXATTN_ERR_ARG;
  if (static_cast<long long>(B) * H * ceil_div(Sq, FLEXATTN_QTILE) * splits > INT_MAX) return FLEXATTN_ERR_OVERFLOW;
  if (use_static) {
    const size_t need = flexattn_decode_workspace_bytes(B, H, Hkv, Sq, D, splits);
    if (need > fa::kStaticScratchBytes) {
      std::snprintf(g_last_error, sizeof(g_last_error),
                    "flexattn_decode_static: %zu bytes of split results exceed the %zu-byte static scratch "
                    "(use fewer splits or flexattn_decode with a workspace)",
                    need, static_cast<size_t>(fa::kStaticScratchBytes));
      return FLEXATTN_ERR_SCRATCH;
    }
  } else if (splits > 1) {
    if (!workspace) return FLEXATTN_ERR_NULLPTR;
    if (!aligned(workspace, 16)) return FLEXATTN_ERR_ALIGN;
    if (workspace_bytes < flexattn_decode_workspace_bytes(B, H, Hkv, Sq, D, splits)) return FLEXATTN_ERR_ARG;
  }

  fa::FwdLaunch p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Skv = Skv;
  p.D = D;
  p.is_fp32 = 0;
  p.mask_kind = mask_kind;
  p.mod_kind = mod_kind;
  fill_variant(p.va, prm, scale, mask_kind, mod_kind);
  {
    const Strides qs = strides_of(prm->q_stride, H, Sq, D), ks = strides_of(prm->k_stride, Hkv, Skv, D);
    const Strides vs = strides_of(prm->v_stride, Hkv, Skv, D), os = strides_of(prm->o_stride, H, Sq, D);
    int ls = check_layout(qs, Sq, D, 2);
    if (!ls) ls = check_layout(ks, Skv, D, 2);
    if (!ls) ls = check_layout(vs, Skv, D, 2);
    if (!ls) ls = check_layout(os, Sq, D, 2);
    if (ls) return ls;
    if (!non_overlapping(os, B, H, Sq, D)) return FLEXATTN_ERR_ARG;
    // packed: the rows of a group's rep query heads are addressed from its
    // first head with 32-bit byte offsets
    if (packed && ((rep - 1) * qs.h + static_cast<long long>(Sq + FLEXATTN_QTILE) * qs.r) * 2 > INT_MAX)
      return FLEXATTN_ERR_OVERFLOW;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FLEXATTN_ERR_ALIGN;
    if (lse && !aligned(lse, 4)) return FLEXATTN_ERR_ALIGN;
    p.q_sb = qs.b; p.q_sh = qs.h; p.q_sr = static_cast<int>(qs.r);
    p.k_sb = ks.b; p.k_sh = ks.h; p.k_sr = static_cast<int>(ks.r);
    p.v_sb = vs.b; p.v_sh = vs.h; p.v_sr = static_cast<int>(vs.r);
    p.o_sb = os.b; p.o_sh = os.h; p.o_sr = static_cast<int>(os.r);
  }
  p.kv_count = block_mask ? block_mask->kv_count : nullptr;
  p.kv_list = block_mask ? block_mask->kv_list : nullptr;
  p.nq = ceil_div(Sq, FLEXATTN_QTILE);
  p.nk = ceil_div(Skv, FLEXATTN_TILE);
  p.bm_num_b = block_mask ? block_mask->num_b : 1;
  p.splits = splits;
  if (splits > 1 && use_static) {
    // the scratch of the device the work runs on: the stream's, which must
    // be the current device (where the address is looked up)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (stream) {
      int sdev = 0;
      e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
      if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
      if (sdev != dev) {
        std::snprintf(g_last_error, sizeof(g_last_error),
                      "flexattn_decode_static: the stream belongs to device %d, the current device is %d",
                      sdev, dev);
        return FLEXATTN_ERR_ARG;
      }
    }
    e = fa::static_scratch(dev, &workspace);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
  }
  if (splits > 1) {
    const size_t rows = static_cast<size_t>(B) * H * Sq;
    p.ws_o = static_cast<float*>(workspace);
    p.ws_lse = p.ws_o + static_cast<size_t>(splits) * rows * D;
  }
  hipError_t e = fa::launch_attn_decode(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return FLEXATTN_OK;
}

}  // namespace

extern "C" {

int flexattn_decode(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                    int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                    const flexattn_params* params, const flexattn_block_mask* block_mask, int splits,
                    void* workspace, size_t workspace_bytes, void* stream) {
  log_begin();
  const int st = decode_impl(q, k, v, out, lse, B, H, Hkv, Sq, Skv, D, scale, mask_kind, mod_kind, params,
                             block_mask, splits, workspace, workspace_bytes, false, stream);
  log_end("flexattn_decode", st, "B=%d H=%d Hkv=%d Sq=%d Skv=%d D=%d %s scale=%g mask=0x%x mod=%d block_mask=%s splits=%d workspace_bytes=%zu stream=%p",
          B, H, Hkv, Sq, Skv, D, dtype_name(params), scale, mask_kind, mod_kind, block_mask ? "given" : "none",
          splits, workspace_bytes, stream);
  return st;
}

int flexattn_decode_static(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                           int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                           const flexattn_params* params, const flexattn_block_mask* block_mask, int splits,
                           void* stream) {
  log_begin();
  const int st = decode_impl(q, k, v, out, lse, B, H, Hkv, Sq, Skv, D, scale, mask_kind, mod_kind, params,
                             block_mask, splits, nullptr, 0, true, stream);
  log_end("flexattn_decode_static", st, "B=%d H=%d Hkv=%d Sq=%d Skv=%d D=%d %s scale=%g mask=0x%x mod=%d block_mask=%s splits=%d stream=%p",
          B, H, Hkv, Sq, Skv, D, dtype_name(params), scale, mask_kind, mod_kind, block_mask ? "given" : "none",
          splits, stream);
  return st;
}

static int bwd_body(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
                    int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                    const flexattn_params* params, const flexattn_block_mask* block_mask,
                    void* stream) {
  const flexattn_params* prm = params ? params : &kDefaultParams;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !delta)
    return FLEXATTN_ERR_NULLPTR;
  int st = check_attn_args(prm, B, H, Hkv, Sq, Skv, D, scale, mask_kind, mod_kind, block_mask);
  if (st) return st;
  if (prm->dtype != FLEXATTN_BF16) return FLEXATTN_ERR_UNSUPPORTED;
  if (ceil_div(Skv, FLEXATTN_TILE) > fa::kPairMaxKeyTiles) return FLEXATTN_ERR_UNSUPPORTED;
  const Strides qs = strides_of(prm->q_stride, H, Sq, D), ks = strides_of(prm->k_stride, Hkv, Skv, D);
  const Strides vs = strides_of(prm->v_stride, Hkv, Skv, D), os = strides_of(prm->o_stride, H, Sq, D);
  {
    int ls = check_layout(qs, Sq, D, 2);
    if (!ls) ls = check_layout(ks, Skv, D, 2);
    if (!ls) ls = check_layout(vs, Skv, D, 2);
    if (!ls) ls = check_layout(os, Sq, D, 2);
    if (ls) return ls;
    // dq, dk and dv take the strides of q, k and v: their elements must be
    // distinct addresses (and out's, which dout shares, for symmetry with
    // the forward that wrote out)
    if (!non_overlapping(qs, B, H, Sq, D) || !non_overlapping(ks, B, Hkv, Skv, D) ||
        !non_overlapping(vs, B, Hkv, Skv, D) || !non_overlapping(os, B, H, Sq, D))
      return FLEXATTN_ERR_ARG;
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return FLEXATTN_ERR_ALIGN;
  if (!aligned(lse, 4) || !aligned(delta, 4)) return FLEXATTN_ERR_ALIGN;

  fa::BwdLaunch p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = delta;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Skv = Skv;
  p.D = D;
  p.mask_kind = mask_kind;
  p.mod_kind = mod_kind;
  p.scale = scale;
  fill_variant(p.va, prm, scale, mask_kind, mod_kind);
  p.kv_count = block_mask ? block_mask->kv_count : nullptr;
  p.kv_list = block_mask ? block_mask->kv_list : nullptr;
  p.nq = ceil_div(Sq, FLEXATTN_QTILE);
  p.nk = ceil_div(Skv, FLEXATTN_TILE);
  p.bm_num_b = block_mask ? block_mask->num_b : 1;
  p.q_sb = qs.b; p.q_sh = qs.h; p.q_sr = static_cast<int>(qs.r);
  p.k_sb = ks.b; p.k_sh = ks.h; p.k_sr = static_cast<int>(ks.r);
  p.v_sb = vs.b; p.v_sh = vs.h; p.v_sr = static_cast<int>(vs.r);
  p.o_sb = os.b; p.o_sh = os.h; p.o_sr = static_cast<int>(os.r);
  hipError_t e = fa::launch_attn_bwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return FLEXATTN_OK;
}

int flexattn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
                 int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                 const flexattn_params* params, const flexattn_block_mask* block_mask,
                 void* stream) {
  log_begin();
  const int st = bwd_body(q, k, v, out, lse, dout, dq, dk, dv, delta, B, H, Hkv, Sq, Skv, D, scale, mask_kind,
                          mod_kind, params, block_mask, stream);
  log_end("flexattn_bwd", st, "B=%d H=%d Hkv=%d Sq=%d Skv=%d D=%d %s scale=%g mask=0x%x mod=%d block_mask=%s stream=%p",
          B, H, Hkv, Sq, Skv, D, dtype_name(params), scale, mask_kind, mod_kind, block_mask ? "given" : "none",
          stream);
  return st;
}

}  // extern "C"
