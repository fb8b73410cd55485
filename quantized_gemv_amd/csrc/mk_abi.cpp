// The C-ABI of libmk: argument validation, the packed-weight and scratch
// layouts, and the launches.  Every entry point is declared, with its
// contract, in include/mk.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstddef>
#include <atomic>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_launch.h"
#include "mk_shared.h"

using namespace mk;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMatQ = 0, kMatK = 1, kMatV = 2, kMatO = 3, kMatGate = 4, kMatUp = 5, kMatDown = 6, kMatEmbed = 7;

size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

struct MatSize {
  size_t codes, scales, tscale;
};

MatSize mat_bytes(uint32_t fmt, size_t N, size_t K, int n_tscale) {
  MatSize s{0, 0, 0};
  if (fmt == FMT_BF16) s.codes = N * K * 2;
  if (fmt == FMT_FP8) { s.codes = N * K; s.scales = N * 4; }
  if (fmt == FMT_FP4) { s.codes = N * K / 2; s.scales = N * K / 16; s.tscale = 4ull * n_tscale; }
  return s;
}

}  // namespace

struct mk_model {
  mk_config cfg;
  uint32_t fmt_lin = FMT_BF16, fmt_down = FMT_BF16, fmt_embed = FMT_BF16;
  Params P;                 // host copy of the kernel parameters
  size_t weights_bytes = 0, algo_bytes = 0, layer_stride = 0;
  size_t scratch_bytes = 0, params_off = 0, tok_off = 0;
  size_t scratch_reported = 0;
  void* d_weights = nullptr;
  void* d_kv = nullptr;
  void* d_rope = nullptr;
  uint8_t* d_scratch = nullptr;
  void* d_trace = nullptr;
  bool bound = false, packed = false, params_dirty = true;
  int device = -1, cus = 0;
  int grid_opt = 0;
  int64_t spin_limit = 100000000;
  std::vector<int32_t> sched;   // the work table (host copy)
  std::vector<int32_t> qkv_word;   // word of each q/k/v row in the per-producer layout
  uint32_t tag_skew = 0;
  uint32_t poll_sleep = 0;
  uint32_t lm_balance = 0;
  int launch_mode = -1;         // 0 cooperative, 1 plain launch of a grid that fits at once, -1 choose
  int split_chunk = 192;        // split attention: cached positions per participant (0: off)
  int split_from = 704;         // split attention from this position on
  int split_n = 0;              // helpers per KV head in the work table
  int coresident = 0;           // decode workgroups the device holds at once (set by mk_bind)
  int fp4_search = 0;           // NVFP4 block scale search radius (0: absolute-maximum recipe)
  int prefill_mode = 0;         // mk_prefill: 0 one decode launch per position, 1 batched (matrix cores)
  int sync_mode = 0;            // 0 tagged exchange words, 1 one grid barrier per phase hand-off
  size_t pf_off = 0;            // batched-prefill workspace in the scratch buffer
  uint32_t epoch = 0;
  uint64_t uid = 0;             // unique per model handle (owner of the static scratch contents)
  bool static_dirty = true;     // parameters changed since they were last put in the static scratch
  Params P_static;              // the parameter block of the no-allocation path (held for its upload)
  std::string err;
};

namespace {

// KV cache bytes: per layer, K then V, per KV head a plane of max_ctx
// (rounded up to 4) positions by head_dim bf16 values.
size_t kv_bytes(const mk_config& c) {
  return (size_t)c.n_layers * 2 * c.n_kv_heads * (size_t)((c.max_ctx + 3) & ~3) * c.head_dim * 2;
}

int fail(mk_model* m, int code, const char* fmt, ...) {
  if (m) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    m->err = buf;
  }
  return code;
}

int hip_fail(mk_model* m, hipError_t e, const char* what) {
  return fail(m, MK_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCK(m, call)                                         \
  do {                                                         \
    hipError_t e_ = (call);                                    \
    if (e_ != hipSuccess) return hip_fail((m), e_, #call);    \
  } while (0)

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

// The largest grid the library launches.
constexpr int kMaxGrid = 1024;

// Ints of the work table for `grid` workgroups and of the q/k/v pair map
// that follows it (per KV head, one word offset per pair of its rows).
size_t sched_ints(const mk_config& c, int grid) {
  return (size_t)grid * kWaves * kSchedInts +
         (size_t)c.n_kv_heads * (c.n_q_heads / c.n_kv_heads + 2) * c.head_dim / 2;
}

// Lay out the weight arena and fill the matrix descriptors.
void layout_weights(mk_model* m) {
  const mk_config& c = m->cfg;
  const size_t H = c.hidden, I = c.intermediate, V = c.vocab, hd = c.head_dim;
  const size_t nq = c.n_q_heads, nkv = c.n_kv_heads, nqkv = (nq + 2 * nkv) * hd;
  size_t off = 0, algo = 0;
  auto place = [&](Mat& mt, uint32_t fmt, size_t N, size_t K, int n_ts) {
    const MatSize s = mat_bytes(fmt, N, K, n_ts);
    mt.fmt = fmt;
    mt.N = (uint32_t)N;
    mt.K = (uint32_t)K;
    mt.codes = off;
    off = align_up(off + s.codes);
    mt.scales = off;
    off = align_up(off + s.scales);
    mt.tscale = off;
    off = align_up(off + s.tscale);
    mt.ts_mode = 0;
    mt.ts_b0 = mt.ts_b1 = 0;
    algo += s.codes + s.scales + s.tscale;
  };
  auto place_vec = [&](uint64_t& o, size_t n) {
    o = off;
    off = align_up(off + n * 2);
    algo += n * 2;
  };
  Params& P = m->P;
  place(P.embed, m->fmt_embed, V, H, 0);
  const size_t layers_begin = off;
  const size_t algo_before = algo;
  Layer& L = P.layer0;
  place(L.qkv, m->fmt_lin, nqkv, H, 3);
  L.qkv.ts_mode = 1;
  L.qkv.ts_b0 = (uint32_t)(nq * hd);
  L.qkv.ts_b1 = (uint32_t)((nq + nkv) * hd);
  place(L.o, m->fmt_lin, H, nq * hd, 1);
  place(L.gu, m->fmt_lin, 2 * I, H, 2);
  L.gu.ts_mode = 2;
  place(L.down, m->fmt_down, H, I, 1);
  place_vec(L.in_norm, H);
  place_vec(L.post_norm, H);
  place_vec(L.q_norm, hd);
  place_vec(L.k_norm, hd);
  m->layer_stride = off - layers_begin;
  const size_t layer_algo = algo - algo_before;
  off = layers_begin + m->layer_stride * c.n_layers;
  algo = algo_before + layer_algo * c.n_layers;
  place_vec(P.final_norm, H);
  P.layer_stride = m->layer_stride;
  // the work table and q/k/v pair map (written at bind), sized for the
  // largest grid
  P.sched = off;
  off = align_up(off + sched_ints(m->cfg, kMaxGrid) * sizeof(int32_t));
  m->weights_bytes = off;
  m->algo_bytes = algo;
}

// Batched prefill workspace: per chunk row the residual, the q/k/v outputs,
// the GEMM input (normed residual or attention output) and the SwiGLU
// output; then the LM head's per-wave maxima.
struct PfLayout {
  size_t x, qkv, a, h, bv, bi, total;
};
PfLayout prefill_layout(const mk_config& c) {
  const size_t C = kPrefillChunk, H = c.hidden, I = c.intermediate, hd = c.head_dim;
  const size_t nq = c.n_q_heads, nkv = c.n_kv_heads;
  PfLayout L;
  L.x = 0;
  L.qkv = align_up(L.x + 4 * C * H);
  L.a = align_up(L.qkv + 4 * C * (nq + 2 * nkv) * hd);
  L.h = align_up(L.a + 2 * C * std::max(H, nq * hd));
  L.bv = align_up(L.h + 2 * C * I);
  L.bi = align_up(L.bv + 4ull * kPrefillHeadGroups * 4);
  L.total = align_up(L.bi + 4ull * kPrefillHeadGroups * 4);
  return L;
}
size_t prefill_workspace(const mk_config& c) { return prefill_layout(c).total; }
// The batched prefill's kernels assume K % 64 == 0 for every matrix (the
// GEMM's K stage), hidden <= 4096 (the LM head's LDS row) and head_dim 64 or
// 128 (the attention's instantiations).
bool prefill_supported(const mk_config& c) {
  const int H = c.hidden, I = c.intermediate, q = c.n_q_heads * c.head_dim;
  return H % 64 == 0 && I % 64 == 0 && q % 64 == 0 && H <= 4096 && (c.head_dim == 64 || c.head_dim == 128);
}

// Lay out the scratch buffer: per-layer exchange vectors, argmax words, the
// error word, the params copy, token slots.
// Words of one split-attention partial: the outputs of the KV head's q heads,
// their maxima and sums, padded to 128 bytes.
uint64_t split_pw(const mk_config& c) {
  const uint64_t gs = c.n_q_heads / c.n_kv_heads;
  return (gs * c.head_dim + 2 * gs + 15) / 16 * 16;
}

// The per-producer layout of the q/k/v vector: XCD slot sl holds the rows
// of KV heads g = sl, sl + 8, ... (each head's q rows, k rows, v rows), dealt
// in even blocks over the slot's GEMV workgroups; block i of the slot starts
// at word base + i * stride.
struct QkvSlot {
  uint64_t n = 0, c = 0, stride = 0, base = 0;
};
void qkv_slots(const mk_config& c, int grid, QkvSlot (&sl)[8], uint64_t* total) {
  const int nkv = c.n_kv_heads, gs = c.n_q_heads / c.n_kv_heads, hd = c.head_dim;
  uint64_t w = 0;
  for (int t = 0; t < 8; ++t) {
    QkvSlot q;
    for (int g = t; g < nkv; g += 8) q.n += (uint64_t)(gs + 2) * hd;
    for (int wg = t; wg < grid; wg += 8)
      if (wg >= nkv) ++q.c;
    if (q.n && q.c) {
      q.stride = (2 * ((q.n / 2 + q.c - 1) / q.c) + 15) / 16 * 16;
      q.base = w;
      w += q.c * q.stride;
    }
    sl[t] = q;
  }
  *total = w;
}

void layout_scratch(mk_model* m, int grid, bool for_sizing = true) {
  const mk_config& c = m->cfg;
  Xch& X = m->P.x;
  const uint64_t H = c.hidden, hd = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads, I = c.intermediate;
  auto al = [](uint64_t w) { return (w + 15) / 16 * 16; };   // 128-byte boundaries
  X.base = 0;
  uint64_t lw = 0;
  const uint64_t pw = split_pw(c);
  uint64_t sizes[kTypes] = {(nq + 2 * nkv) * hd, nkv * (uint64_t)kMaxSplit * pw, nq * hd / 2, H, I / 2, H};
  // the residuals and the SwiGLU output in the per-producer layout: the
  // GEMV workgroups' blocks (even length) each start a 128-byte line
  const uint32_t cg = (uint32_t)std::max(grid - (int)nkv, 1);
  for (int t : {(int)V_XO, (int)V_H, (int)V_XD}) {
    const uint64_t np = sizes[t] / 2;
    const uint32_t stride = (uint32_t)((2 * ((np + cg - 1) / cg) + 15) / 16 * 16);
    X.pad_c[t] = cg;
    X.pad_stride[t] = stride;
    sizes[t] = (uint64_t)cg * stride;
  }
  for (int t : {(int)V_QKV, (int)V_ATT, (int)V_O}) X.pad_c[t] = X.pad_stride[t] = 0;
  {
    QkvSlot sl[8];
    qkv_slots(c, grid, sl, &sizes[V_QKV]);
  }
  for (int t = 0; t < kTypes; ++t) {
    X.off[t] = lw;
    lw = al(lw + sizes[t]);
  }
  X.layer_words = lw;
  uint64_t w = lw * (uint64_t)c.n_layers;
  X.arg = al(w);
  w = X.arg + 4ull * grid;   // per workgroup: argmax value and index, LM-head ticks, rows and XCD
  X.bar = al(w);
  w = X.bar + 5ull * c.n_layers + 1;
  X.err = al(w);
  X.amax = X.err + 1;
  w = X.amax + 1;
  w = (w + 31) / 32 * 32;   // 256-byte boundary
  X.words = w;
  m->params_off = align_up(w * 8);
  m->tok_off = align_up(m->params_off + sizeof(Params));
  m->pf_off = align_up(m->tok_off + 4ull * ((size_t)c.max_ctx + 4));
  m->scratch_bytes = align_up(m->pf_off + prefill_workspace(c));
  if (for_sizing) m->scratch_reported = m->scratch_bytes;
}

// The work table: which workgroup runs which KV head's attention, and which
// rows of each matrix every compute wave owns.  Returns an error message, or
// nullptr.
//  * Attention: KV head g on workgroup g, which the hardware places on XCD
//    g % 8 (workgroups are dealt to the XCDs round robin).
//  * Every matrix is split into contiguous blocks of rows, one block per
//    workgroup, so one workgroup's output words share cache lines only with
//    each other (words of many producers in one line make every exchange
//    slower); inside a block the rows go to the compute waves in turn.
//  * QKV: the q, k and v rows of head g go to the other workgroups of the
//    same XCD, so the attention workgroup gathers them from its own L2.
//  * O, gate/up (units of four rows = one output word), down: over the
//    workgroups without attention; each matrix starts at a different wave
//    so every wave gets a similar share.
const char* build_sched(const mk_config& c, int grid, std::vector<int32_t>& tab, int* split_n = nullptr,
                        std::vector<int32_t>* qkv_word = nullptr) {
  const int nkv = c.n_kv_heads, hd = c.head_dim, nq = c.n_q_heads, gs = nq / nkv;
  const int H = c.hidden, I = c.intermediate;
  const int nA = nkv;
  if (grid < nA + 1) return "grid too small for one attention workgroup per KV head";
  tab.assign((size_t)grid * kWaves * kSchedInts, -1);
  auto hdr = [&](int wg, int i) -> int32_t& { return tab[(size_t)wg * kWaves * kSchedInts + i]; };
  auto unit = [&](int wg, int cw, int i) -> int32_t& {
    return tab[(size_t)wg * kWaves * kSchedInts + (size_t)(cw + 1) * kSchedInts + i];
  };
  auto add = [&](int wg, int cw, int off, int maxu, int row) -> bool {
    for (int k = 0; k < maxu; ++k)
      if (unit(wg, cw, off + k) < 0) {
        unit(wg, cw, off + k) = row;
        return true;
      }
    return false;
  };
  // units [0, n) of `rows` in contiguous blocks over `wgs`, waves in turn
  // from `w0`; with `even`, the blocks have even bounds (the per-producer
  // exchange layout deals word pairs)
  auto deal = [&](const std::vector<int>& rows, const std::vector<int>& wgs, int w0, int slot, int maxu,
                  bool even = false) -> bool {
    const size_t n = rows.size(), C = wgs.size();
    for (size_t i = 0; i < C; ++i) {
      const size_t a = even ? 2 * (n / 2 * i / C) : n * i / C, b = even ? 2 * (n / 2 * (i + 1) / C) : n * (i + 1) / C;
      for (size_t u = a; u < b; ++u)
        if (!add(wgs[i], (int)((w0 + (u - a)) % kCW), slot, maxu, rows[u])) return false;
    }
    return true;
  };
  for (int wg = 0; wg < grid; ++wg) hdr(wg, S_ATT) = wg < nA ? wg : -1;
  // QKV, per XCD slot, in the per-producer layout; the table after the
  // workgroups' rows maps each KV head's q/k/v pairs to their words
  QkvSlot qs[8];
  uint64_t qtotal = 0;
  qkv_slots(c, grid, qs, &qtotal);
  const size_t np_head = (size_t)(gs + 2) * hd / 2;
  tab.resize((size_t)grid * kWaves * kSchedInts + nkv * np_head, -1);
  int32_t* qmap = tab.data() + (size_t)grid * kWaves * kSchedInts;
  std::vector<int32_t> word((size_t)(nq + 2 * nkv) * hd, -1);
  for (int sl = 0; sl < 8; ++sl) {
    std::vector<int> wgs;
    for (int wg = sl; wg < grid; wg += 8)
      if (wg >= nA) wgs.push_back(wg);
    std::vector<int> rows;
    for (int g = sl; g < nkv; g += 8) {
      for (int i = 0; i < gs * hd; ++i) rows.push_back(g * gs * hd + i);
      for (int i = 0; i < hd; ++i) rows.push_back((nq + g) * hd + i);
      for (int i = 0; i < hd; ++i) rows.push_back((nq + nkv + g) * hd + i);
    }
    if (rows.empty()) continue;
    if (wgs.empty()) return "no workgroup on an XCD that holds a KV head";
    if (!deal(rows, wgs, 0, S_QKV, kMaxQKV, true)) return "too many QKV rows per wave for this grid";
    const QkvSlot& q = qs[sl];
    for (size_t u = 0; u < rows.size(); ++u)
      word[rows[u]] = (int32_t)(q.base + xpad_word((uint32_t)u, (uint32_t)q.n, (uint32_t)q.c, (uint32_t)q.stride));
    size_t hu = 0;   // the slot's heads in deal order
    for (int g = sl; g < nkv; g += 8, hu += 2 * np_head)
      for (size_t j = 0; j < np_head; ++j)
        qmap[(size_t)g * np_head + j] = (int32_t)(q.base + xpad_word((uint32_t)(hu + 2 * j), (uint32_t)q.n,
                                                                      (uint32_t)q.c, (uint32_t)q.stride));
  }
  for (int wg = 0; wg < grid; ++wg)
    for (int cw = 0; cw < kCW; ++cw)
      for (int k = 0; k < kMaxQKV; ++k) {
        const int r = unit(wg, cw, S_QKV + k);
        unit(wg, cw, S_QKVW + k) = r >= 0 ? word[r] : -1;
      }
  if (qkv_word) *qkv_word = word;
  // O, gate/up, down
  std::vector<int> gw;
  for (int wg = nA; wg < grid; ++wg) gw.push_back(wg);
  std::vector<int> rh(H), ri(I / 2);
  for (int i = 0; i < H; ++i) rh[i] = i;
  for (int i = 0; i < I / 2; ++i) ri[i] = i;
  if (!deal(rh, gw, 0, S_O, kMaxO, true)) return "too many O rows per wave for this grid";
  if (!deal(ri, gw, 0, S_GU, kMaxGU, true)) return "too many gate/up units per wave for this grid";
  if (!deal(rh, gw, 3, S_D, kMaxD, true)) return "too many down rows per wave for this grid";
  // split attention: the GEMV workgroups of an XCD that holds KV heads help
  // those heads (in turn), up to the partials the home holds in LDS
  const int cap = kMaxSplit;
  std::vector<int> helpers(nkv, 0);
  for (int sl = 0; sl < 8; ++sl) {
    std::vector<int> heads;
    for (int g = sl; g < nkv; g += 8) heads.push_back(g);
    if (heads.empty()) continue;
    int idx = 0;
    for (int wg = sl; wg < grid; wg += 8) {
      if (wg < nA) continue;
      const int g = heads[idx % heads.size()], i = idx / (int)heads.size() + 1;
      ++idx;
      if (i > cap) continue;
      hdr(wg, S_SPLIT) = g;
      hdr(wg, S_SPLIT_IDX) = i;
      helpers[g] = std::max(helpers[g], i);
    }
  }
  if (split_n) *split_n = *std::min_element(helpers.begin(), helpers.end());
  // per-workgroup inputs, in the courier's order: xd, qkv, o, xo, h (with
  // split attention: xd, qkv, the helped head's q, o, xo, h)
  for (int wg = 0; wg < grid; ++wg) {
    bool q = false, o = false, gu = false, d = false;
    for (int cw = 0; cw < kCW; ++cw) {
      q |= unit(wg, cw, S_QKV) >= 0;
      o |= unit(wg, cw, S_O) >= 0;
      gu |= unit(wg, cw, S_GU) >= 0;
      d |= unit(wg, cw, S_D) >= 0;
    }
    const bool att = hdr(wg, S_ATT) >= 0;
    const bool need[5] = {q || o, att, o, gu || d, d};
    const int slot[5] = {S_IXD, S_IQKV, S_IO, S_IXO, S_IH};
    int n = 0;
    for (int i = 0; i < 5; ++i) hdr(wg, slot[i]) = need[i] ? n++ : -1;
    hdr(wg, S_NIN) = n;
    n = need[0] + need[1];
    hdr(wg, S_IQS_L) = hdr(wg, S_SPLIT) >= 0 ? n++ : -1;
    hdr(wg, S_IO_L) = need[2] ? n++ : -1;
    hdr(wg, S_IXO_L) = need[3] ? n++ : -1;
    hdr(wg, S_IH_L) = need[4] ? n++ : -1;
    hdr(wg, S_NIN_L) = n;
    hdr(wg, S_FLAGS) = (need[0] ? 1 : 0) | (o ? 2 : 0) | (need[3] ? 4 : 0) | (d ? 8 : 0);
  }
  return nullptr;
}

int n_phases(const mk_config& c) { return 6 * c.n_layers + 4; }

// Before mk_bind the compute-unit count is unknown, so sizes are reported for
// the grid option if set, else for the largest grid the library launches.
int sizing_grid(const mk_model* m) { return m->grid_opt > 0 ? m->grid_opt : kMaxGrid; }

int validate_cfg(const mk_config* c) {
  if (!c) return MK_E_INVALID;
  if (c->n_layers <= 0 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->intermediate <= 0 || c->vocab <= 0 || c->max_ctx <= 0 || !(c->rope_theta > 0) || !(c->rms_eps > 0))
    return MK_E_INVALID;
  if (c->wfmt < MK_WFMT_BF16 || c->wfmt > MK_WFMT_FP4_MIX) return MK_E_INVALID;
  if (c->n_q_heads % c->n_kv_heads) return MK_E_UNSUPPORTED;
  if (!decode_shape_supported(c->head_dim, c->n_q_heads / c->n_kv_heads, c->hidden, c->n_q_heads * c->head_dim,
                              c->intermediate))
    return MK_E_UNSUPPORTED;
  if (c->hidden % 128 || c->intermediate % 16 || (c->n_q_heads * c->head_dim) % 16) return MK_E_UNSUPPORTED;
  if (c->hidden > 4096 || c->intermediate / 2 > 6144 || c->n_q_heads * c->head_dim / 2 > 6144)
    return MK_E_UNSUPPORTED;
  if (c->n_layers > kMaxLayers || c->max_ctx > (1 << 20)) return MK_E_UNSUPPORTED;
  return MK_OK;
}

// Grids the kernel handles: at most kMaxGrid workgroups and a work table
// within the per-wave unit limits.
int check_grid(mk_model* m, int grid) {
  if (grid < 1) return fail(m, MK_E_INVALID, "grid must be positive");
  std::vector<int32_t> tab;
  const char* why = build_sched(m->cfg, grid, tab);
  if (why) return fail(m, MK_E_UNSUPPORTED, "grid %d: %s", grid, why);
  return MK_OK;
}

// Fill the kernel parameters that depend on the grid and the bound buffers,
// and upload them.
void fill_params(mk_model* m) {
  const mk_config& c = m->cfg;
  Params& P = m->P;
  // C-style casts: in the device pass of this file these fields are global pointers
  P.w = (decltype(P.w))m->d_weights;
  P.w_bytes = (uint32_t)m->weights_bytes;
  P.kv = (decltype(P.kv))m->d_kv;
  P.rope = (decltype(P.rope))m->d_rope;
  P.xch = (decltype(P.xch))m->d_scratch;
  P.trace = m->d_trace;
  P.L = c.n_layers;
  P.H = c.hidden;
  P.nq = c.n_q_heads;
  P.nkv = c.n_kv_heads;
  P.hd = c.head_dim;
  P.I = c.intermediate;
  P.V = c.vocab;
  P.max_ctx = c.max_ctx;
  P.eps = c.rms_eps;
  P.spin_limit = (uint64_t)m->spin_limit;
  P.tag_skew = m->tag_skew;
  P.poll_sleep = m->poll_sleep;
  P.lm_balance = m->lm_balance;
  P.n_phases = n_phases(c);
  P.split_max = kMaxSplit;
  P.split_pw = (int)split_pw(c);
  P.bar_fence = m->sync_mode == 2 ? 1u : 0u;
}

int sync_params(mk_model* m, hipStream_t s) {
  if (!m->params_dirty) return MK_OK;
  fill_params(m);
  HIPCK(m, hipMemcpyAsync(m->d_scratch + m->params_off, &m->P, sizeof(Params), hipMemcpyHostToDevice, s));
  HIPCK(m, hipStreamSynchronize(s));  // the host copy is a stack-independent member, but keep ordering simple
  m->params_dirty = false;
  return MK_OK;
}

int32_t read_token_and_error(mk_model* m, const int32_t* d_next, hipStream_t s) {
  int32_t tok = -1;
  uint32_t err = 0;
  HIPCK(m, hipMemcpyAsync(&tok, d_next, 4, hipMemcpyDeviceToHost, s));
  HIPCK(m, hipMemcpyAsync(&err, m->d_scratch + 8 * m->P.x.err, 4, hipMemcpyDeviceToHost, s));
  HIPCK(m, hipStreamSynchronize(s));
  if (err) {
    uint32_t zero = 0;
    HIPCK(m, hipMemcpy(m->d_scratch + 8 * m->P.x.err, &zero, 4, hipMemcpyHostToDevice));
    // a step that failed may have left workgroups short of some barriers:
    // restart the grid-barrier counters
    HIPCK(m, launch_zero_words(reinterpret_cast<uint64_t*>(m->d_scratch) + m->P.x.bar, 5ull * m->cfg.n_layers + 1,
                               s));
    HIPCK(m, hipStreamSynchronize(s));
    if (err & 1u) return fail(m, MK_E_TIMEOUT, "a kernel wait exceeded its spin bound");
    return fail(m, MK_E_INVALID, "the kernel read a token outside the vocabulary");
  }
  return tok;
}

// Helpers per KV head of split attention at position `pos` (0: none).
int split_helpers(const mk_model* m, int pos) {
  const bool barrier = m->sync_mode != 0;
  return !barrier && m->split_chunk > 0 && pos >= m->split_from ? std::min(m->split_n, pos / m->split_chunk) : 0;
}

// One decode launch of `nsteps` greedy steps from position `pos` with the
// parameter block at `dp` (device memory) and exchange tags of epochs
// epoch .. epoch + nsteps - 1.  A launch of more than one step has no
// split-attention helpers at any of its positions.
int launch_with(mk_model* m, const Params* dp, uint32_t epoch, const int32_t* d_token, int pos, int32_t* d_next,
                float* d_logits, hipStream_t s, int nsteps = 1) {
  const mk_config& c = m->cfg;
  const bool coop = m->launch_mode == 0 || (m->launch_mode < 0 && m->P.grid > m->coresident);
  const bool barrier = m->sync_mode != 0;
  const int ns = split_helpers(m, pos);
  if (nsteps > 1 && (ns > 0 || split_helpers(m, pos + nsteps - 1) > 0))
    return fail(m, MK_E_INVALID, "a launch of %d steps from position %d would use split attention", nsteps, pos);
  if (!coop && m->P.grid > m->coresident)
    return fail(m, MK_E_UNSUPPORTED, "plain launch: grid %d exceeds the %d workgroups the device holds at once",
                m->P.grid, m->coresident);
  HIPCK(m, launch_decode(dp, c.wfmt, c.head_dim, c.n_q_heads / c.n_kv_heads, c.hidden, c.n_q_heads * c.head_dim,
                         c.intermediate, m->P.grid, coop, barrier, d_token, pos, nsteps, ns, epoch, d_next, d_logits,
                         s));
  return MK_OK;
}

int launch_step(mk_model* m, const int32_t* d_token, int pos, int32_t* d_next, float* d_logits, hipStream_t s) {
  int rc = sync_params(m, s);
  if (rc) return rc;
  m->epoch = (m->epoch + 1) & kEpochMask;
  if (m->epoch == 0) {  // tags would repeat: clear the exchange words and restart
    HIPCK(m, launch_zero_words(reinterpret_cast<uint64_t*>(m->d_scratch), m->P.x.err, s));
    m->epoch = 1;
  }
  const Params* dp = reinterpret_cast<const Params*>(m->d_scratch + m->params_off);
  return launch_with(m, dp, m->epoch, d_token, pos, d_next, d_logits, s);
}

// n greedy steps from position `pos` in as few launches as the exchange
// epochs and split attention allow: a launch never lets the epoch wrap and
// runs at most kMaxStepsPerLaunch steps, and a position with split-attention
// helpers gets a launch of its own (a helper reads KV rows another CU wrote;
// only a kernel boundary makes those visible to it).  A later launch reads
// its first token from the previous one's last output, on the same stream.
constexpr int kMaxStepsPerLaunch = 512;
int launch_steps(mk_model* m, const int32_t* d_token, int pos, int n, int32_t* d_next, float* d_logits,
                 hipStream_t s) {
  int rc = sync_params(m, s);
  if (rc) return rc;
  const Params* dp = reinterpret_cast<const Params*>(m->d_scratch + m->params_off);
  for (int done = 0; done < n;) {
    uint32_t e = (m->epoch + 1) & kEpochMask;
    if (e == 0) {   // tags would repeat: clear the exchange words and restart
      HIPCK(m, launch_zero_words(reinterpret_cast<uint64_t*>(m->d_scratch), m->P.x.err, s));
      e = 1;
    }
    const int p0 = pos + done, ns0 = split_helpers(m, p0);
    const int cap = (int)std::min<uint64_t>({(uint64_t)(n - done), (uint64_t)kMaxStepsPerLaunch,
                                              (uint64_t)kEpochMask - e + 1});
    int k = 1;
    while (ns0 == 0 && k < cap && split_helpers(m, p0 + k) == 0) ++k;
    rc = launch_with(m, dp, e, done == 0 ? d_token : d_next + done - 1, p0, d_next + done,
                     d_logits ? d_logits + (size_t)done * m->cfg.vocab : nullptr, s, k);
    if (rc) return rc;
    m->epoch = e + (uint32_t)k - 1;
    done += k;
  }
  return MK_OK;
}

// ---- the no-allocation step (mk_decode_step_async_noalloc)
// Its scratch (exchange words, argmax words, error word and the kernel
// parameter block, laid out as in the bound scratch buffer) is this
// file-scope device array.  Each device holds its own copy, at the address
// hipGetSymbolAddress reports with that device current; the array's name in
// host code is only a handle for that lookup.
constexpr size_t kStaticScratchBytes = 32ull << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Per device: the array's device address, the exchange epoch of the last
// step run in it (tags stay unique across every model that uses the array),
// which model's parameters it holds, and how much of it any
// model has used.
struct StaticSlot {
  uint8_t* ptr = nullptr;
  uint32_t epoch = 0;
  uint64_t owner = 0;
  size_t extent = 0;
};
std::mutex g_static_mu;
std::vector<StaticSlot> g_static;
std::atomic<uint64_t> g_next_uid{1};

// Bytes of the static array one step of this model uses.
size_t static_need(const mk_model* m) { return m->params_off + sizeof(Params); }

}  // namespace

extern "C" {

int mk_create(const mk_config* cfg, mk_model** out) {
  if (!out) return MK_E_INVALID;
  *out = nullptr;
  const int v = validate_cfg(cfg);
  if (v) return v;
  mk_model* m = new (std::nothrow) mk_model();
  if (!m) return MK_E_INVALID;
  m->cfg = *cfg;
  m->uid = g_next_uid.fetch_add(1);
  std::memset(&m->P, 0, sizeof(Params));
  if (cfg->wfmt == MK_WFMT_FP8_ROW) m->fmt_lin = m->fmt_down = m->fmt_embed = FMT_FP8;
  if (cfg->wfmt == MK_WFMT_FP4_MIX) {
    m->fmt_lin = FMT_FP4;
    m->fmt_down = m->fmt_embed = FMT_FP8;
  }
  layout_weights(m);
  layout_scratch(m, sizing_grid(m));
  if (m->weights_bytes > kMaxBuffer || 8 * m->P.x.words > kMaxBuffer) {
    delete m;
    return MK_E_UNSUPPORTED;   // the kernels address weights and scratch with 32-bit offsets
  }
  *out = m;
  return MK_OK;
}

int mk_query_sizes(const mk_model* m, mk_sizes* out) {
  if (!m || !out) return MK_E_INVALID;
  const mk_config& c = m->cfg;
  out->weights = m->weights_bytes;
  out->kv = kv_bytes(c);
  out->rope = (size_t)c.max_ctx * (c.head_dim / 2) * 2 * 4;
  out->scratch = m->scratch_reported;
  out->trace = mk_has_xray() ? sizeof(mk_trace_rec) * (size_t)sizing_grid(m) * n_phases(c) : 0;
  out->weight_bytes_per_token = m->algo_bytes;
  out->kv_bytes_per_position = (size_t)c.n_layers * 2 * c.n_kv_heads * c.head_dim * 2;
  return MK_OK;
}

int mk_bind(mk_model* m, void* d_weights, void* d_kv, void* d_rope, void* d_scratch, void* d_trace,
            mk_stream_t stream) {
  if (!m) return MK_E_INVALID;
  if (!d_weights || !d_kv || !d_rope || !d_scratch)
    return fail(m, MK_E_INVALID, "mk_bind: a required buffer is null");
  if (!aligned(d_weights) || !aligned(d_kv) || !aligned(d_rope) || !aligned(d_scratch) ||
      (d_trace && !aligned(d_trace)))
    return fail(m, MK_E_INVALID, "mk_bind: buffers must be 256-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  HIPCK(m, hipGetDevice(&m->device));
  hipDeviceProp_t prop;
  HIPCK(m, hipGetDeviceProperties(&prop, m->device));
  int coop = 0;
  HIPCK(m, hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, m->device));
  if (!coop) return fail(m, MK_E_UNSUPPORTED, "device lacks cooperative launch");
  m->cus = prop.multiProcessorCount;
  const int grid = m->grid_opt > 0 ? m->grid_opt : m->cus;
  if (grid > kMaxGrid) return fail(m, MK_E_UNSUPPORTED, "grid %d above %d", grid, kMaxGrid);
  const int gc = check_grid(m, grid);
  if (gc) return gc;
  {
    const mk_config& c = m->cfg;
    int per_cu = 0;
    HIPCK(m, decode_coresident(c.wfmt, c.head_dim, c.n_q_heads / c.n_kv_heads, c.hidden, c.n_q_heads * c.head_dim,
                               c.intermediate, &per_cu));
    m->coresident = per_cu * m->cus;
  }
  layout_scratch(m, grid, false);
  if (m->scratch_bytes > m->scratch_reported)
    return fail(m, MK_E_UNSUPPORTED, "grid %d needs %zu scratch bytes, more than the %zu reported", grid,
                m->scratch_bytes, m->scratch_reported);
  m->P.grid = grid;
  m->d_weights = d_weights;
  m->d_kv = d_kv;
  m->d_rope = d_rope;
  m->d_scratch = static_cast<uint8_t*>(d_scratch);
  m->d_trace = mk_has_xray() ? d_trace : nullptr;
  m->bound = true;
  m->params_dirty = true;
  m->static_dirty = true;
  m->epoch = 0;
  const char* why = build_sched(m->cfg, grid, m->sched, &m->split_n, &m->qkv_word);
  if (why) return fail(m, MK_E_UNSUPPORTED, "grid %d: %s", grid, why);
  HIPCK(m, hipMemsetAsync(d_scratch, 0, m->scratch_bytes, s));
  // the attention reads whole 4-position V tiles (weight 0 past the last
  // cached position): never-written slots must hold finite values
  HIPCK(m, hipMemsetAsync(d_kv, 0, kv_bytes(m->cfg), s));
  m->P.qmap = m->P.sched + (uint64_t)grid * kWaves * kSchedInts * sizeof(int32_t);
  HIPCK(m, hipMemcpyAsync(static_cast<uint8_t*>(d_weights) + m->P.sched, m->sched.data(),
                          m->sched.size() * sizeof(int32_t), hipMemcpyHostToDevice, s));
  return sync_params(m, s);
}

int mk_pack_weights(mk_model* m, const void* const* d_tensors, int32_t n_tensors, mk_stream_t stream) {
  if (!m) return MK_E_INVALID;
  const mk_config& c = m->cfg;
  if (!d_tensors || n_tensors != 2 + 11 * c.n_layers)
    return fail(m, MK_E_INVALID, "mk_pack_weights: expected %d tensors", 2 + 11 * c.n_layers);
  for (int i = 0; i < n_tensors; ++i)
    if (!d_tensors[i]) return fail(m, MK_E_INVALID, "mk_pack_weights: tensor %d is null", i);
  if (!m->bound) return fail(m, MK_E_STATE, "mk_pack_weights before mk_bind");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* W = static_cast<uint8_t*>(m->d_weights);
  uint32_t* amax = reinterpret_cast<uint32_t*>(m->d_scratch + 8 * m->P.x.amax);
  auto T = [&](int i) { return static_cast<const uint16_t*>(d_tensors[i]); };
  // one source matrix [N,K] into rows row_off + r*row_step of `mt`
  auto pack = [&](const uint16_t* src, const Mat& mt, size_t layer_off, int N, int K, int row_off, int row_step,
                  int ts_index) -> hipError_t {
    uint8_t* codes = W + mt.codes + layer_off;
    if (mt.fmt == FMT_BF16)
      return launch_pack_bf16(src, N, K, reinterpret_cast<uint16_t*>(codes), row_off, row_step, s);
    if (mt.fmt == FMT_FP8)
      return launch_pack_fp8(src, N, K, codes, reinterpret_cast<float*>(W + mt.scales + layer_off), row_off,
                             row_step, s);
    return launch_pack_fp4(src, N, K, codes, W + mt.scales + layer_off,
                           reinterpret_cast<float*>(W + mt.tscale + layer_off), ts_index, amax, row_off, row_step,
                           m->fp4_search, s);
  };
  auto copy_vec = [&](const uint16_t* src, uint64_t off, size_t n) -> hipError_t {
    return hipMemcpyAsync(W + off, src, n * 2, hipMemcpyDeviceToDevice, s);
  };
  const int H = c.hidden, I = c.intermediate, hd = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const Layer& L = m->P.layer0;
  HIPCK(m, pack(T(0), m->P.embed, 0, c.vocab, H, 0, 1, 0));
  for (int l = 0; l < c.n_layers; ++l) {
    const int b = 1 + 11 * l;
    const size_t lo = (size_t)l * m->layer_stride;
    HIPCK(m, copy_vec(T(b + 0), L.in_norm + lo, H));
    HIPCK(m, pack(T(b + 1), L.qkv, lo, nq * hd, H, 0, 1, 0));
    HIPCK(m, pack(T(b + 2), L.qkv, lo, nkv * hd, H, nq * hd, 1, 1));
    HIPCK(m, pack(T(b + 3), L.qkv, lo, nkv * hd, H, (nq + nkv) * hd, 1, 2));
    HIPCK(m, copy_vec(T(b + 4), L.q_norm + lo, hd));
    HIPCK(m, copy_vec(T(b + 5), L.k_norm + lo, hd));
    HIPCK(m, pack(T(b + 6), L.o, lo, H, nq * hd, 0, 1, 0));
    HIPCK(m, copy_vec(T(b + 7), L.post_norm + lo, H));
    HIPCK(m, pack(T(b + 8), L.gu, lo, I, H, 0, 2, 0));
    HIPCK(m, pack(T(b + 9), L.gu, lo, I, H, 1, 2, 1));
    HIPCK(m, pack(T(b + 10), L.down, lo, H, I, 0, 1, 0));
  }
  HIPCK(m, copy_vec(T(1 + 11 * c.n_layers), m->P.final_norm, H));
  HIPCK(m, launch_rope(static_cast<float*>(m->d_rope), c.max_ctx, hd, (double)c.rope_theta, s));
  HIPCK(m, hipStreamSynchronize(s));
  m->packed = true;
  return MK_OK;
}

int mk_read_packed(mk_model* m, int32_t layer, int32_t matrix, void* h_codes, void* h_scales,
                   void* h_block_scales, float* h_tensor_scale) {
  if (!m) return MK_E_INVALID;
  const mk_config& c = m->cfg;
  if (matrix < 0 || matrix > kMatEmbed || !h_codes) return fail(m, MK_E_INVALID, "mk_read_packed: bad matrix");
  if (matrix != kMatEmbed && (layer < 0 || layer >= c.n_layers))
    return fail(m, MK_E_INVALID, "mk_read_packed: bad layer");
  if (!m->packed) return fail(m, MK_E_STATE, "mk_read_packed before mk_pack_weights");
  const int H = c.hidden, I = c.intermediate, hd = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const Layer& L = m->P.layer0;
  const size_t lo = matrix == kMatEmbed ? 0 : (size_t)layer * m->layer_stride;
  const Mat* mt = nullptr;
  int N = 0, K = 0, row_off = 0, row_step = 1, ts_index = 0;
  switch (matrix) {
    case kMatQ: mt = &L.qkv; N = nq * hd; K = H; break;
    case kMatK: mt = &L.qkv; N = nkv * hd; K = H; row_off = nq * hd; ts_index = 1; break;
    case kMatV: mt = &L.qkv; N = nkv * hd; K = H; row_off = (nq + nkv) * hd; ts_index = 2; break;
    case kMatO: mt = &L.o; N = H; K = nq * hd; break;
    case kMatGate: mt = &L.gu; N = I; K = H; row_step = 2; break;
    case kMatUp: mt = &L.gu; N = I; K = H; row_off = 1; row_step = 2; ts_index = 1; break;
    case kMatDown: mt = &L.down; N = H; K = I; break;
    default: mt = &m->P.embed; N = c.vocab; K = H; break;
  }
  const uint8_t* W = static_cast<const uint8_t*>(m->d_weights);
  size_t row_bytes = mt->fmt == FMT_BF16 ? 2ull * K : (mt->fmt == FMT_FP8 ? (size_t)K : (size_t)K / 2);
  HIPCK(m, hipMemcpy2D(h_codes, row_bytes, W + mt->codes + lo + row_bytes * row_off, row_bytes * row_step,
                       row_bytes, N, hipMemcpyDeviceToHost));
  if (mt->fmt == FMT_FP8) {
    if (!h_scales) return fail(m, MK_E_INVALID, "mk_read_packed: h_scales is null");
    HIPCK(m, hipMemcpy2D(h_scales, 4, W + mt->scales + lo + 4ull * row_off, 4ull * row_step, 4, N,
                         hipMemcpyDeviceToHost));
  } else if (mt->fmt == FMT_FP4) {
    if (!h_block_scales || !h_tensor_scale) return fail(m, MK_E_INVALID, "mk_read_packed: FP4 outputs are null");
    const size_t bsb = K / 16;
    HIPCK(m, hipMemcpy2D(h_block_scales, bsb, W + mt->scales + lo + bsb * row_off, bsb * row_step, bsb, N,
                         hipMemcpyDeviceToHost));
    HIPCK(m, hipMemcpy(h_tensor_scale, W + mt->tscale + lo + 4ull * ts_index, 4, hipMemcpyDeviceToHost));
  }
  return MK_OK;
}

int mk_decode_step_async(mk_model* m, const int32_t* d_token, int32_t pos, int32_t* d_next, float* d_logits,
                         mk_stream_t stream) {
  if (!m) return MK_E_INVALID;
  if (!d_token || !d_next || d_token == d_next)
    return fail(m, MK_E_INVALID, "mk_decode_step_async: token buffers must be distinct and non-null");
  if (pos < 0 || pos >= m->cfg.max_ctx) return fail(m, MK_E_INVALID, "position %d outside [0, %d)", pos, m->cfg.max_ctx);
  if (!m->bound || !m->packed) return fail(m, MK_E_STATE, "decode before mk_bind and mk_pack_weights");
  return launch_step(m, d_token, pos, d_next, d_logits, reinterpret_cast<hipStream_t>(stream));
}

int mk_decode_steps_async(mk_model* m, const int32_t* d_token, int32_t pos, int32_t n, int32_t* d_next,
                          float* d_logits, mk_stream_t stream) {
  if (!m) return MK_E_INVALID;
  if (!d_token || !d_next) return fail(m, MK_E_INVALID, "mk_decode_steps_async: token buffers must be non-null");
  if (n < 1) return fail(m, MK_E_INVALID, "mk_decode_steps_async: %d steps", n);
  if (d_token >= d_next && d_token < d_next + n)
    return fail(m, MK_E_INVALID, "mk_decode_steps_async: d_token lies inside d_next[0..n)");
  if (pos < 0 || (int64_t)pos + n > m->cfg.max_ctx)
    return fail(m, MK_E_INVALID, "positions %d..%d outside [0, %d)", pos, pos + n - 1, m->cfg.max_ctx);
  if (!m->bound || !m->packed) return fail(m, MK_E_STATE, "decode before mk_bind and mk_pack_weights");
  return launch_steps(m, d_token, pos, n, d_next, d_logits, reinterpret_cast<hipStream_t>(stream));
}

int mk_decode_step_async_noalloc(mk_model* m, const int32_t* d_token, int32_t pos, int32_t* d_next,
                                 float* d_logits, mk_stream_t stream) {
  if (!m) return MK_E_INVALID;
  if (!d_token || !d_next || d_token == d_next)
    return fail(m, MK_E_INVALID, "mk_decode_step_async_noalloc: token buffers must be distinct and non-null");
  if (pos < 0 || pos >= m->cfg.max_ctx) return fail(m, MK_E_INVALID, "position %d outside [0, %d)", pos, m->cfg.max_ctx);
  if (!m->bound || !m->packed) return fail(m, MK_E_STATE, "decode before mk_bind and mk_pack_weights");
  if (m->sync_mode != 0)
    return fail(m, MK_E_UNSUPPORTED, "mk_decode_step_async_noalloc: the grid-barrier variant (option 11) needs the "
                                     "bound scratch buffer");
  if (static_need(m) > kStaticScratchBytes)
    return fail(m, MK_E_UNSUPPORTED,
                "mk_decode_step_async_noalloc: this model's step needs %zu bytes of scratch, more than the "
                "library's static %zu",
                static_need(m), (size_t)kStaticScratchBytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  HIPCK(m, hipGetDevice(&dev));
  if (dev != m->device)
    return fail(m, MK_E_INVALID, "mk_decode_step_async_noalloc: device %d is current, the model is bound on %d", dev,
                m->device);
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static.size() <= (size_t)dev) g_static.resize((size_t)dev + 1);
  StaticSlot& slot = g_static[(size_t)dev];
  if (!slot.ptr) {   // first use on this device: look up this device's copy of the array
    void* p = nullptr;
    HIPCK(m, hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    slot.ptr = static_cast<uint8_t*>(p);
  }
  if (slot.owner != m->uid || m->static_dirty) {
    // this model's parameter block (exchange base = the array) and work table
    fill_params(m);
    m->P_static = m->P;
    m->P_static.xch = (decltype(m->P_static.xch))slot.ptr;
    HIPCK(m, hipMemcpyAsync(slot.ptr + m->params_off, &m->P_static, sizeof(Params), hipMemcpyHostToDevice, s));
    slot.owner = m->uid;
    slot.extent = std::max(slot.extent, (size_t)(8 * m->P.x.err));
    m->static_dirty = false;
  }
  uint32_t epoch = (slot.epoch + 1) & kEpochMask;
  if (epoch == 0) {   // tags would repeat: clear every exchange word used so far
    HIPCK(m, launch_zero_words(reinterpret_cast<uint64_t*>(slot.ptr), slot.extent / 8, s));
    epoch = 1;
  }
  slot.epoch = epoch;
  // a failed earlier step leaves its code in the error word: start clean
  HIPCK(m, launch_zero_words(reinterpret_cast<uint64_t*>(slot.ptr) + m->P.x.err, 1, s));
  return launch_with(m, reinterpret_cast<const Params*>(slot.ptr + m->params_off), epoch, d_token, pos, d_next,
                     d_logits, s);
}

int32_t mk_decode_step(mk_model* m, int32_t token, int32_t pos, mk_stream_t stream) {
  if (!m) return MK_E_INVALID;
  if (token < 0 || token >= m->cfg.vocab) return fail(m, MK_E_INVALID, "token %d outside the vocabulary", token);
  if (pos < 0 || pos >= m->cfg.max_ctx) return fail(m, MK_E_INVALID, "position %d outside [0, %d)", pos, m->cfg.max_ctx);
  if (!m->bound || !m->packed) return fail(m, MK_E_STATE, "decode before mk_bind and mk_pack_weights");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t* tok = reinterpret_cast<int32_t*>(m->d_scratch + m->tok_off);
  HIPCK(m, hipMemcpyAsync(tok, &token, 4, hipMemcpyHostToDevice, s));
  int rc = launch_step(m, tok, pos, tok + 1, nullptr, s);
  if (rc) return rc;
  return read_token_and_error(m, tok + 1, s);
}

// Positions 0..n-1 through every layer in chunks of kPrefillChunk (matrix
// products on the matrix cores), then the LM head of position n-1 and its
// argmax into d_next (and its logits into d_logits when non-null).
int prefill_batched(mk_model* m, const int32_t* d_prompt, int n, int32_t* d_next, float* d_logits, hipStream_t s) {
  const mk_config& c = m->cfg;
  {
    const int rc = sync_params(m, s);
    if (rc) return rc;
  }
  const PfLayout Lo = prefill_layout(c);
  uint8_t* ws = m->d_scratch + m->pf_off;
  const Params* dp = reinterpret_cast<const Params*>(m->d_scratch + m->params_off);
  const char* dl = reinterpret_cast<const char*>(dp) + offsetof(Params, layer0);
  PrefillArgs a;
  a.params = dp;
  a.mat_qkv = reinterpret_cast<const Mat*>(dl + offsetof(Layer, qkv));
  a.mat_o = reinterpret_cast<const Mat*>(dl + offsetof(Layer, o));
  a.mat_gu = reinterpret_cast<const Mat*>(dl + offsetof(Layer, gu));
  a.mat_down = reinterpret_cast<const Mat*>(dl + offsetof(Layer, down));
  a.fmt_lin = m->P.layer0.qkv.fmt;
  a.fmt_down = m->P.layer0.down.fmt;
  a.layer_stride = m->P.layer_stride;
  a.in_norm = m->P.layer0.in_norm;
  a.post_norm = m->P.layer0.post_norm;
  a.L = c.n_layers;
  a.H = c.hidden;
  a.hd = c.head_dim;
  a.nq = c.n_q_heads;
  a.nkv = c.n_kv_heads;
  a.I = c.intermediate;
  a.X = reinterpret_cast<float*>(ws + Lo.x);
  a.QKV = reinterpret_cast<float*>(ws + Lo.qkv);
  a.A = reinterpret_cast<uint16_t*>(ws + Lo.a);
  a.Hb = reinterpret_cast<uint16_t*>(ws + Lo.h);
  a.best_v = reinterpret_cast<float*>(ws + Lo.bv);
  a.best_i = reinterpret_cast<int32_t*>(ws + Lo.bi);
  a.next = d_next;
  a.logits = d_logits;
  for (int c0 = 0; c0 < n; c0 += kPrefillChunk) {
    a.c0 = c0;
    a.cn = std::min(kPrefillChunk, n - c0);
    a.last = c0 + a.cn == n;
    a.tokens = d_prompt + c0;
    HIPCK(m, launch_prefill_chunk(a, s));
  }
  return MK_OK;
}

int32_t mk_prefill(mk_model* m, const int32_t* h_tokens, int32_t n, mk_stream_t stream) {
  if (!m) return MK_E_INVALID;
  if (!h_tokens || n <= 0 || n > m->cfg.max_ctx) return fail(m, MK_E_INVALID, "mk_prefill: bad prompt length %d", n);
  for (int i = 0; i < n; ++i)
    if (h_tokens[i] < 0 || h_tokens[i] >= m->cfg.vocab)
      return fail(m, MK_E_INVALID, "mk_prefill: token %d outside the vocabulary", i);
  if (!m->bound || !m->packed) return fail(m, MK_E_STATE, "prefill before mk_bind and mk_pack_weights");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t* tok = reinterpret_cast<int32_t*>(m->d_scratch + m->tok_off);
  int32_t* prompt = tok + 2;
  HIPCK(m, hipMemcpyAsync(prompt, h_tokens, 4ull * n, hipMemcpyHostToDevice, s));
  if (m->prefill_mode == 1) {
    const int rc = prefill_batched(m, prompt, n, tok + 1, nullptr, s);
    if (rc) return rc;
    return read_token_and_error(m, tok + 1, s);
  }
  for (int i = 0; i < n; ++i) {
    int rc = launch_step(m, prompt + i, i, tok + 1, nullptr, s);
    if (rc) return rc;
  }
  return read_token_and_error(m, tok + 1, s);
}

int mk_check_device_error(mk_model* m, mk_stream_t stream) {
  if (!m) return MK_E_INVALID;
  if (!m->bound) return fail(m, MK_E_STATE, "not bound");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int32_t* next = reinterpret_cast<const int32_t*>(m->d_scratch + m->tok_off) + 1;
  const int32_t r = read_token_and_error(m, next, s);
  return r < 0 ? r : MK_OK;
}

int mk_get_trace(mk_model* m, mk_trace_rec* h_out, size_t cap, size_t* n_out) {
  if (!m || !n_out) return MK_E_INVALID;
  if (!mk_has_xray() || !m->d_trace) {
    *n_out = 0;
    return MK_OK;
  }
  const size_t n = (size_t)m->P.grid * n_phases(m->cfg);
  *n_out = n;
  if (!h_out || cap < n) return fail(m, MK_E_INVALID, "mk_get_trace: need room for %zu records", n);
  HIPCK(m, hipDeviceSynchronize());
  HIPCK(m, hipMemcpy(h_out, m->d_trace, n * sizeof(mk_trace_rec), hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_read_exchange(mk_model* m, int32_t layer, int32_t vec, float* h_out, size_t n) {
  if (!m) return MK_E_INVALID;
  const mk_config& c = m->cfg;
  if (layer < 0 || layer >= c.n_layers) return fail(m, MK_E_INVALID, "mk_read_exchange: bad layer");
  static const int kType[5] = {V_QKV, V_O, V_XO, V_H, V_XD};
  static const bool kPairs[5] = {false, true, false, true, false};
  if (vec < 0 || vec > 4) return fail(m, MK_E_INVALID, "mk_read_exchange: bad vector");
  const size_t len = vec == 0 ? (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim
                   : vec == 1 ? (size_t)c.n_q_heads * c.head_dim
                   : vec == 3 ? (size_t)c.intermediate : (size_t)c.hidden;
  if (!h_out || n != len) return fail(m, MK_E_INVALID, "mk_read_exchange: need %zu outputs", len);
  if (!m->bound || m->epoch == 0) return fail(m, MK_E_STATE, "mk_read_exchange before any decode step");
  const size_t words = kPairs[vec] ? len / 2 : len;
  const Xch& X = m->P.x;
  const int ty = kType[vec];
  const size_t span = ty == V_QKV ? (size_t)(X.off[V_QKV + 1] - X.off[V_QKV])
                     : X.pad_c[ty] ? (size_t)X.pad_c[ty] * X.pad_stride[ty] : words;
  std::vector<uint64_t> raw(span), w(words);
  const uint64_t first = X.base + (uint64_t)layer * X.layer_words + X.off[ty];
  HIPCK(m, hipMemcpy(raw.data(), m->d_scratch + 8 * first, 8 * span, hipMemcpyDeviceToHost));
  for (size_t i = 0; i < words; ++i)
    w[i] = raw[ty == V_QKV ? (size_t)m->qkv_word[i]
                           : xpad_word((uint32_t)i, (uint32_t)words, X.pad_c[ty], X.pad_stride[ty])];
  const uint32_t tag = (m->epoch << kPhaseBits) | (uint32_t)(2 + kTypes * layer + kType[vec]);
  for (size_t i = 0; i < words; ++i) {
    if ((uint32_t)w[i] != tag)
      return fail(m, MK_E_STATE, "mk_read_exchange: word %zu was not written by the last step", i);
    const uint32_t pay = (uint32_t)(w[i] >> 32);
    if (kPairs[vec]) {
      const uint32_t lo = pay << 16, hi = pay & 0xFFFF0000u;
      memcpy(&h_out[2 * i], &lo, 4);
      memcpy(&h_out[2 * i + 1], &hi, 4);
    } else {
      memcpy(&h_out[i], &pay, 4);
    }
  }
  return MK_OK;
}

int mk_decode_codes(int32_t codec, const uint8_t* d_codes, int32_t n, float* d_out, mk_stream_t stream) {
  if (codec < 0 || codec > 4 || n < 0 || (n > 0 && (!d_codes || !d_out))) return MK_E_INVALID;
  const hipError_t e = launch_decode_codes(codec, d_codes, n, d_out, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? MK_OK : MK_E_HIP;
}

int mk_set_option(mk_model* m, int32_t key, int64_t value) {
  if (!m) return MK_E_INVALID;
  switch (key) {
    case 0:
      if (value < 0) return fail(m, MK_E_INVALID, "grid %lld out of range", (long long)value);
      if (m->bound) return fail(m, MK_E_STATE, "set the grid before mk_bind");
      if (value > kMaxGrid) return fail(m, MK_E_INVALID, "grid above %d", kMaxGrid);
      m->grid_opt = (int)value;
      layout_scratch(m, sizing_grid(m));
      break;
    case 3:
      if (value < 0) return fail(m, MK_E_INVALID, "spin limit must be >= 0");
      m->spin_limit = value;
      break;
    case 4:
      if (value < 0 || value > 0xFFFF) return fail(m, MK_E_INVALID, "tag skew out of range");
      m->tag_skew = (uint32_t)value;
      break;
    case 5:
      if (value < 0 || value > 16) return fail(m, MK_E_INVALID, "poll back-off out of range");
      m->poll_sleep = (uint32_t)value;
      break;
    case 12:
      if (value < 0 || value > 1) return fail(m, MK_E_INVALID, "LM-head balancing must be 0 or 1");
      m->lm_balance = (uint32_t)value;
      break;
    case 6:
      if (value < -1 || value > 1) return fail(m, MK_E_INVALID, "launch mode must be -1, 0 or 1");
      m->launch_mode = (int)value;
      break;
    case 7:
      if (value < 0 || value > (1 << 20)) return fail(m, MK_E_INVALID, "split chunk out of range");
      m->split_chunk = (int)value;
      break;
    case 8:
      if (value < 0 || value > (1 << 20)) return fail(m, MK_E_INVALID, "split start position out of range");
      m->split_from = (int)value;
      break;
    case 10:
      if (value < 0 || value > 1) return fail(m, MK_E_INVALID, "prefill mode must be 0 or 1");
      if (value == 1 && !prefill_supported(m->cfg)) return fail(m, MK_E_UNSUPPORTED, "batched prefill: shape not supported");
      m->prefill_mode = (int)value;
      break;
    case 11:
      if (value < 0 || value > 2) return fail(m, MK_E_INVALID, "sync mode must be 0, 1 or 2");
      m->sync_mode = (int)value;
      break;
    case 9:
      if (value < 0 || value > 0x7E) return fail(m, MK_E_INVALID, "FP4 scale search radius out of range");
      if (m->packed) return fail(m, MK_E_STATE, "set the FP4 scale search before mk_pack_weights");
      m->fp4_search = (int)value;
      break;
    default:
      return fail(m, MK_E_INVALID, "unknown option %d", key);
  }
  m->params_dirty = true;
  m->static_dirty = true;
  return MK_OK;
}

int mk_has_xray(void) {
#ifdef MK_XRAY
  return 1;
#else
  return 0;
#endif
}

const char* mk_status_str(int status) {
  switch (status) {
    case MK_OK: return "ok";
    case MK_E_INVALID: return "invalid argument";
    case MK_E_UNSUPPORTED: return "unsupported shape or format";
    case MK_E_STATE: return "call out of order";
    case MK_E_HIP: return "HIP runtime error";
    case MK_E_TIMEOUT: return "kernel wait timed out";
    default: return "unknown status";
  }
}

const char* mk_last_error(const mk_model* m) { return m ? m->err.c_str() : "null model"; }

void mk_destroy(mk_model* m) { delete m; }

}  // extern "C"
