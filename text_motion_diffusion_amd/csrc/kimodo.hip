// C ABI of the gfx950 denoiser library (declarations and semantics in
// include/kimodo.h). Host side: argument validation, workspace layout, weight
// conversion, the enqueue of one DDIM step (root transformer -> global-to-local
// root -> body transformer -> CFG + DDIM; Kimodo WebGPU README, "Architecture"
// diagram) and the sampling loop, which replays one captured HIP graph per step
// with the per-step scalars read on the device at a step counter.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "kimodo.h"

using kmd::f16;

namespace {

constexpr int D = 1024, H = 8, F = 2048, ROOT = 5, BODY = 274, FEATS = ROOT + BODY, TEXT = 4096;
constexpr int KPAD_ROOT = 64, KPAD_BODY = 320;  // input-projection K padded to a multiple of the GEMM k-tile
constexpr int LAYER_TENSORS = 12, HEAD_TENSORS = 8, TAIL_TENSORS = 2;
// Split-K partial sums of the small GEMMs: one region per concurrent chain.
constexpr size_t SPLITK_FLOATS = size_t(1) << 22;
constexpr int MAX_CHAINS_LAYOUT = 2;

bool config_ok(const kimodo_config *c) {
  if (!c) return false;
  if (c->d_model != D || c->n_heads != H || c->d_ff != F || c->root_feats != ROOT || c->body_feats != BODY ||
      c->text_dim != TEXT)
    return false;
  if (c->layers_root < 0 || c->layers_root > 256 || c->layers_body < 0 || c->layers_body > 256) return false;
  if (c->max_batch < 1 || c->max_batch > 512 || c->max_frames < 1 || c->max_frames > 4096) return false;
  if (c->max_steps < 1 || c->max_steps > 1000) return false;
  return c->dtype == KIMODO_F32 || c->dtype == KIMODO_BF16 || c->dtype == KIMODO_F16;
}

int tensors_per_net(int layers) { return HEAD_TENSORS + LAYER_TENSORS * layers + TAIL_TENSORS; }
int weight_count(const kimodo_config &c) { return tensors_per_net(c.layers_root) + tensors_per_net(c.layers_body); }

// Shape of canonical weight `index` (cols = 0 for vectors).
void weight_shape(const kimodo_config &c, int index, int64_t *rows, int64_t *cols) {
  int net = 0, i = index;
  if (i >= tensors_per_net(c.layers_root)) {
    net = 1;
    i -= tensors_per_net(c.layers_root);
  }
  const int L = net ? c.layers_body : c.layers_root;
  const int64_t k_in = net ? FEATS : ROOT, n_out = net ? BODY : ROOT;
  static const int64_t head[HEAD_TENSORS][2] = {{D, TEXT}, {D, 0}, {D, D}, {D, 0}, {D, D}, {D, 0}, {D, -1}, {D, 0}};
  static const int64_t layer[LAYER_TENSORS][2] = {{3 * D, D}, {3 * D, 0}, {D, D}, {D, 0}, {D, 0}, {D, 0},
                                                  {F, D},     {F, 0},     {D, F}, {D, 0}, {D, 0}, {D, 0}};
  if (i < HEAD_TENSORS) {
    *rows = head[i][0];
    *cols = head[i][1] < 0 ? k_in : head[i][1];
  } else if (i < HEAD_TENSORS + LAYER_TENSORS * L) {
    const int j = (i - HEAD_TENSORS) % LAYER_TENSORS;
    *rows = layer[j][0];
    *cols = layer[j][1];
  } else {
    *rows = n_out;
    *cols = i == HEAD_TENSORS + LAYER_TENSORS * L ? D : 0;
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Key positions of a sequence of T frames rounded up to the attention key block.
int seq_pad(int T) { return ((T + 2 + 63) / 64) * 64; }
// Packed token rows a sequence of T frames can take: T + 2 rounded up to 8.
int seq_rows(int T) { return (T + 2 + 7) & ~7; }

// Where the kernels read weight i from: the caller's tensor, or its converted
// copy in the workspace (matrices -> compute type, vectors -> fp32).
struct WeightPlan {
  std::vector<size_t> off;  // workspace offset of the converted copy, SIZE_MAX = use the caller's tensor
  std::vector<size_t> n;
  std::vector<bool> matrix;
  size_t bytes = 0;
};

WeightPlan plan_weights(const kimodo_config &c) {
  WeightPlan w;
  const int n = weight_count(c);
  w.off.assign(n, SIZE_MAX);
  w.n.resize(n);
  w.matrix.resize(n);
  for (int i = 0; i < n; ++i) {
    int64_t r, k;
    weight_shape(c, i, &r, &k);
    w.matrix[i] = k > 0;
    w.n[i] = (size_t)r * (k > 0 ? k : 1);
    size_t bytes = 0;
    if (w.matrix[i] && c.dtype == KIMODO_BF16) bytes = w.n[i] * 2;
    if (!w.matrix[i] && c.dtype != KIMODO_F32) bytes = w.n[i] * 4;
    if (bytes) {
      w.off[i] = w.bytes;
      w.bytes += align256(bytes);
    }
  }
  return w;
}

// Workspace layout: every buffer 256-byte aligned, in a fixed order.
struct Layout {
  size_t h, h1, qkv, vt, attn, tmp, ffn, a_in, proj, head_root, head_body, state, known, kmask, splitk, pe, sin_feat,
      t_hidden, ttok[2], txtok[2], text_act, in_pad[2], coef, steps, lengths, counter, bad_weights, tok, mot, tok_g,
      row_ps, weights, total;
};

Layout plan(const kimodo_config &c) {
  const size_t e = c.dtype == KIMODO_F32 ? 4 : 2;
  const size_t Bm = c.max_batch, Tm = c.max_frames, Sm = c.max_steps;
  const size_t M = 2 * Bm * seq_rows((int)Tm), MF = 2 * Bm * Tm;
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.h = take(M * D * e);
  L.h1 = take(M * D * e);
  L.qkv = take(M * 3 * D * e);
  L.vt = take(2 * Bm * D * seq_pad(Tm) * e);
  L.attn = take(M * D * e);
  L.tmp = take(M * D * e);
  L.ffn = take(M * F * e);
  L.a_in = take(MF * KPAD_BODY * e);
  L.proj = take(MF * D * 4);
  L.head_root = take(M * ROOT * 4);
  L.head_body = take(M * BODY * 4);
  L.state = take(Bm * Tm * FEATS * 4);
  L.known = take(Bm * Tm * FEATS * 4);
  L.kmask = take(Bm * Tm * FEATS);
  L.splitk = take(MAX_CHAINS_LAYOUT * SPLITK_FLOATS * 4);
  L.pe = take((Tm + 2) * D * 4);
  L.sin_feat = take(Sm * D * e);
  L.t_hidden = take(Sm * D * e);
  for (int n = 0; n < 2; ++n) L.ttok[n] = take(Sm * D * e);
  for (int n = 0; n < 2; ++n) L.txtok[n] = take(2 * Bm * D * e);
  L.text_act = take(2 * Bm * TEXT * e);
  L.in_pad[0] = take((size_t)D * KPAD_ROOT * e);
  L.in_pad[1] = take((size_t)D * KPAD_BODY * e);
  L.coef = take(Sm * 2 * 4);
  L.steps = take(Sm * 4);
  L.lengths = take(Bm * 4);
  L.counter = take(4);
  L.bad_weights = take(4);
  // token-row packing of a chain (at most 2 Bm sequences of at most Tm + 2 tokens)
  L.tok = take((2 * Bm + 1) * 4);
  L.mot = take((2 * Bm + 1) * 4);
  L.tok_g = take(2 * Bm * 4);
  L.row_ps = take(M * 4);
  L.weights = take(plan_weights(c).bytes);
  L.total = off;
  return L;
}

struct LayerW {
  const void *qkvW, *oW, *ff1W, *ff2W;
  const float *qkvb, *ob, *ln1g, *ln1b, *ff1b, *ff2b, *ln2g, *ln2b;
};
struct NetW {
  const void *txtW, *t1W, *t2W, *inW, *outW;
  const float *txtb, *t1b, *t2b, *inb, *outb;
  std::vector<LayerW> layers;
  void *in_pad;
  int k_in, kpad, n_out;
};

// A weight tensor's set-up pass: converted into dst, or (dst null: the
// kernels read the caller's tensor) only checked to be finite.
struct Conversion {
  const void *src;
  void *dst;
  size_t n;
  bool to_f16;
};

}  // namespace

// A captured step graph with its key. done is recorded after the graph's last
// replay and waited on before the graph is destroyed.
struct StepGraph {
  int B = -1, T = -1;
  float w = 0.f;
  bool constrained = false;
  std::vector<int32_t> len;  // the clip lengths: they fix the packed row counts
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t done = nullptr;
  bool done_recorded = false;
  uint64_t last_use = 0;
};
// Step graphs kept per ctx (least recently used one replaced): enough for a
// timeline's free first segment and constrained later ones at two lengths.
constexpr int GRAPH_SLOTS = 4;

// Kernel chains of one step: the two guidance groups. (Splitting each group
// further into halves of the clips measured slower at 16, 32 and 128 clips.)
constexpr int MAX_CHAINS = 2;
// Up to this many packed token rows (both guidance groups: twice the sum over
// clips of length + 2 rounded up to 8) a step runs both groups as one chain:
// every launch of so small a step is latency-bound, and one chain has half the
// launches of two (1 clip of 150 frames: 2.63 -> 2.51 ms per step; 4 takes of
// 90 frames: 2.88 -> 2.71 ms). From 16 clips of 150 frames (4,864 rows) two
// concurrent chains are faster (4.25 against 4.35 ms). The rows, not B and T,
// decide: a clip padded to a longer T then runs exactly as at its own length.
constexpr int MERGE_MAX_ROWS = 2048;
static_assert(MAX_CHAINS <= MAX_CHAINS_LAYOUT, "one split-K region per chain");

struct kimodo_ctx {
  kimodo_config cfg;
  char *ws;
  Layout L;
  NetW net[2];
  std::vector<Conversion> conversions;
  bool initialized = false;
  bool weights_bad = false;  // set-up found a weight that is not finite in the compute type
  hipStream_t cap_stream = nullptr;
  // extra streams of the concurrent kernel chains (chain 0 runs on the caller's or the capture stream)
  hipStream_t chain_stream[MAX_CHAINS - 1] = {};
  hipEvent_t fork_event = nullptr, join_event[MAX_CHAINS - 1] = {};
  StepGraph graphs[GRAPH_SLOTS];
  uint64_t graph_clock = 0;
  int64_t graph_instantiations = 0, graph_updates = 0;
  std::string err;
  std::vector<int32_t> h_len, h_steps;
  std::vector<float> h_coef;
  // packing of the current call: chain-local token-row offsets, staging
  // offsets, global token rows per sequence, and a chain's row counts
  std::vector<int32_t> h_tok, h_mot, h_tok_g;
  int m_tok = 0, m_mot = 0;
  std::vector<hipEvent_t> events;  // pool for kimodo_profile_step

  template <typename P> P *at(size_t off) { return reinterpret_cast<P *>(ws + off); }
};

namespace {

kimodo_status fail(kimodo_ctx *ctx, kimodo_status s, const std::string &msg) {
  if (ctx) ctx->err = msg;
  return s;
}

#define KMD_HIP(ctx, call)                                                                                      \
  do {                                                                                                          \
    hipError_t e_ = (call);                                                                                     \
    if (e_ != hipSuccess) return fail(ctx, KIMODO_EHIP, std::string(hipGetErrorString(e_)) + " in " + #call); \
  } while (0)

// Device set-up of c's weights and tables, enqueued on s with no host wait:
// every weight converted into the workspace (or, when the kernels read the
// caller's tensor directly, only checked), with the bad_weights flag set if a
// converted value is not finite; the input projections zero-padded to the
// k-tile; the position table; the activation buffers zeroed.
template <typename T>
kimodo_status setup_tables(kimodo_ctx *c, hipStream_t s) {
  const int src_type = c->cfg.dtype == KIMODO_F32 ? 0 : c->cfg.dtype == KIMODO_BF16 ? 1 : 2;
  int32_t *bad = c->at<int32_t>(c->L.bad_weights);
  KMD_HIP(c, kmd::set_int(bad, 0, s));
  for (const Conversion &cv : c->conversions) {
    if (cv.to_f16)
      KMD_HIP(c, kmd::convert_f16(cv.src, src_type, static_cast<f16 *>(cv.dst), cv.n, bad, s));
    else
      KMD_HIP(c, kmd::convert_f32(cv.src, src_type, static_cast<float *>(cv.dst), cv.n, bad, s));
  }
  for (int n = 0; n < 2; ++n) {
    NetW &w = c->net[n];
    KMD_HIP(c, kmd::pad_cols<T>(static_cast<const T *>(w.inW), D, w.k_in, static_cast<T *>(w.in_pad), w.kpad, s));
  }
  KMD_HIP(c, kmd::sinusoid<float>(nullptr, c->cfg.max_frames + 2, c->at<float>(c->L.pe), s));
  // Nothing reads these zeros into a live token: attention gives key
  // positions past a sequence's end exact zeros and never reads its dead rows.
  // They only keep the arithmetic on dead rows finite.
  KMD_HIP(c, kmd::fill_zero<T>(c->at<T>(c->L.vt), (size_t)2 * c->cfg.max_batch * D * seq_pad(c->cfg.max_frames), s));
  const size_t rows = (size_t)2 * c->cfg.max_batch * seq_rows(c->cfg.max_frames);
  KMD_HIP(c, kmd::fill_zero<T>(c->at<T>(c->L.h), rows * D, s));
  KMD_HIP(c, kmd::fill_zero<T>(c->at<T>(c->L.attn), rows * D, s));
  return KIMODO_OK;
}

template <typename T>
kimodo_status init_device(kimodo_ctx *c, hipStream_t s) {
  if (c->initialized) return KIMODO_OK;
  if (!c->cap_stream) KMD_HIP(c, hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
  for (int j = 0; j < MAX_CHAINS - 1; ++j) {
    if (!c->chain_stream[j]) KMD_HIP(c, hipStreamCreateWithFlags(&c->chain_stream[j], hipStreamNonBlocking));
    if (!c->join_event[j]) KMD_HIP(c, hipEventCreateWithFlags(&c->join_event[j], hipEventDisableTiming));
  }
  if (!c->fork_event) KMD_HIP(c, hipEventCreateWithFlags(&c->fork_event, hipEventDisableTiming));
  for (StepGraph &g : c->graphs)
    if (!g.done) KMD_HIP(c, hipEventCreateWithFlags(&g.done, hipEventDisableTiming));
  if (c->weights_bad) return fail(c, KIMODO_EWEIGHTS, "a weight is not finite in the compute type");
  kimodo_status st = setup_tables<T>(c, s);
  if (st != KIMODO_OK) return st;
  int32_t bad_h = 0;
  KMD_HIP(c, hipMemcpyAsync(&bad_h, c->at<int32_t>(c->L.bad_weights), sizeof(int32_t), hipMemcpyDeviceToHost, s));
  KMD_HIP(c, hipStreamSynchronize(s));
  if (bad_h) {
    c->weights_bad = true;
    return fail(c, KIMODO_EWEIGHTS, "a weight is not finite in the compute type (bf16 -> fp16 needs |w| <= 65504)");
  }
  c->initialized = true;
  return KIMODO_OK;
}

// Timestep tokens for rows 0..rows-1 of the device timestep table and text
// tokens of the 2B guidance rows, for both sub-networks.
template <typename T>
kimodo_status conditioning_tokens(kimodo_ctx *c, int B, const float *text, int rows, hipStream_t s) {
  const Layout &L = c->L;
  T *txt = c->at<T>(L.text_act), *sf = c->at<T>(L.sin_feat), *th = c->at<T>(L.t_hidden);
  kmd::GemmAux sk;  // runs on s alone: the first chain's split-K region
  sk.partial = c->at<float>(L.splitk);
  sk.partial_cap = SPLITK_FLOATS;
  KMD_HIP(c, kmd::text_rows<T>(text, B, txt, s));
  KMD_HIP(c, kmd::sinusoid<T>(c->at<int32_t>(L.steps), rows, sf, s));
  for (int n = 0; n < 2; ++n) {
    const NetW &w = c->net[n];
    KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_TXT, txt, TEXT, (const T *)w.txtW, TEXT, w.txtb, c->at<T>(L.txtok[n]), D, 2 * B,
                            D, TEXT, s, sk));
    KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_TMLP1, sf, D, (const T *)w.t1W, D, w.t1b, th, D, rows, D, D, s, sk));
    KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_TMLP2, th, D, (const T *)w.t2W, D, w.t2b, c->at<T>(L.ttok[n]), D, rows, D, D,
                            s, sk));
  }
  return KIMODO_OK;
}

// Both sub-networks for one chain of a DDIM step: guidance group `half` (0:
// the conditional rows p = b, 1: the unconditional rows p = B + b) of clips
// b0 .. b0 + nb - 1, or with groups = 2 (half = 0, b0 = 0, nb = B) both groups
// in one chain of P = 2B sequences. Chains touch disjoint rows of every
// activation buffer and are independent until the CFG combine; sequence p0 +
// q of a chain is clip b0 + q % nb. Within its region (starting at token row
// p0 seq_rows(T)) a chain's token rows are packed: c->m_tok of them, sequence
// q's tokens at rows tok[q] .., each sequence starting on a multiple of 8 rows,
// and its frames at motion rows mot[q] .. (the workspace tables built by
// upload_tables for this B, T and these lengths).
template <typename T>
kimodo_status enqueue_group(kimodo_ctx *c, int B, int T_, int half, int b0, int nb, int groups,
                            const float *x_t_all, const float *known_all, const uint8_t *kmask_all,
                            const kimodo_trace *tr, hipStream_t s) {
  const Layout &L = c->L;
  const int P = groups * nb;  // sequences in this chain
  const int S = T_ + 2, M = c->m_tok, MF = c->m_mot;  // packed token rows, motion rows
  const size_t p0 = (size_t)half * B + b0;
  // first token row / motion row of the chain, and its first row in dense traces
  const size_t r0 = p0 * seq_rows(T_), f0 = p0 * T_, rt = p0 * S;
  const float *x_t = x_t_all + (size_t)b0 * T_ * FEATS;
  const float *known = known_all ? known_all + (size_t)b0 * T_ * FEATS : nullptr;
  const uint8_t *kmask = kmask_all ? kmask_all + (size_t)b0 * T_ * FEATS : nullptr;
  T *h = c->at<T>(L.h) + r0 * D, *h1 = c->at<T>(L.h1) + r0 * D, *attn = c->at<T>(L.attn) + r0 * D;
  T *qkv = c->at<T>(L.qkv) + r0 * 3 * D, *tmp = c->at<T>(L.tmp) + r0 * D, *ffn = c->at<T>(L.ffn) + r0 * F;
  const int S_pad = seq_pad(T_);
  T *vt = c->at<T>(L.vt) + p0 * D * S_pad;
  // the chain's longest sequence (its clips' lengths + 2): the attention
  // kernels size their work by it
  int S_max = 0;
  for (int q = 0; q < nb; ++q) S_max = std::max(S_max, c->h_len[b0 + q] + 2);
  // fp16 sequences of up to 160 tokens: QKV projection and attention in one
  // kernel per (sequence, head), Q/K/V kept in LDS. Below 16 sequences that is
  // under 128 workgroups, each walking all of K with one k-tile in flight; the
  // QKV projection on few-tile GEMM tiles and the attention kernel spread the
  // same work wider (8 sequences of 92 tokens: 2.45 -> 2.17 ms per pass).
  const bool fused_attention = sizeof(T) == 2 && S_max <= 160 && P >= 16;
  // this chain's split-K partial sums (chains run concurrently)
  kmd::GemmAux sk;
  // a two-group chain has both chains' regions
  sk.partial = c->at<float>(L.splitk) + (size_t)half * SPLITK_FLOATS;
  sk.partial_cap = (size_t)groups * SPLITK_FLOATS;
  const int32_t *tok = c->at<int32_t>(L.tok), *mot = c->at<int32_t>(L.mot);
  kmd::GemmAux qkv_aux;
  qkv_aux.vt = vt;
  qkv_aux.seq_pad = S_pad;
  qkv_aux.pk.tok = tok;
  qkv_aux.pk.mot = mot;
  qkv_aux.pk.row_ps = c->at<int32_t>(L.row_ps);
  qkv_aux.partial = sk.partial;
  qkv_aux.partial_cap = sk.partial_cap;
  float *proj = c->at<float>(L.proj) + f0 * D;
  float *head[2] = {c->at<float>(L.head_root) + r0 * ROOT, c->at<float>(L.head_body) + r0 * BODY};
  int32_t *counter = c->at<int32_t>(L.counter);
  const size_t all_rows_bytes = (size_t)2 * B * S * D * sizeof(T);  // one traced layer, all rows
  int layer_index = 0;
  for (int n = 0; n < 2; ++n) {
    const NetW &nw = c->net[n];
    // Row f0 at the widest pitch: the root (64) and body (320) inputs of one
    // chain share its region, and the chains' regions must not overlap.
    T *a_in = c->at<T>(L.a_in) + f0 * KPAD_BODY;
    if (n == 0)
      KMD_HIP(c, kmd::gather_root<T>(x_t, nb, P, T_, mot, a_in, nw.kpad, s));
    else
      KMD_HIP(c, kmd::g2l_gather<T>(head[0], x_t, known, kmask, nb, P, T_, tok, mot, a_in, nw.kpad,
                                    tr && tr->local_root ? tr->local_root + f0 * ROOT : nullptr, s));
    KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_IN, a_in, nw.kpad, (const T *)nw.in_pad, nw.kpad, nw.inb, proj, D, MF, D,
                            nw.kpad, s, sk));
    KMD_HIP(c, kmd::assemble_tokens<T>(proj, c->at<T>(L.ttok[n]), counter, c->at<T>(L.txtok[n]) + p0 * D,
                                       c->at<float>(L.pe), h, P, T_, tok, mot, s));
    if (tr && tr->inputs)  // dense [2][2B][T + 2][1024] copy of the assembled tokens, padded tokens 0
      KMD_HIP(c, kmd::unpack_rows(h, D * (int)sizeof(T), tok, mot, P, 0, S,
                                  static_cast<char *>(tr->inputs) + n * all_rows_bytes + rt * D * sizeof(T), s));
    for (const LayerW &lw : nw.layers) {
      if (fused_attention) {
        KMD_HIP(c, kmd::qkv_attention(reinterpret_cast<const kmd::f16 *>(h),
                                      reinterpret_cast<const kmd::f16 *>(lw.qkvW), lw.qkvb,
                                      reinterpret_cast<kmd::f16 *>(attn), tok, mot, P, S_max, s));
      } else {
        KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_QKV, h, D, (const T *)lw.qkvW, D, lw.qkvb, qkv, 3 * D, M, 3 * D, D, s,
                                qkv_aux));
        KMD_HIP(c, kmd::attention<T>(qkv, vt, attn, tok, mot, P, S_max, S_pad, s));
      }
      // Projections feeding a residual: with split-K the partial sums go
      // straight into the add + LayerNorm kernel, which also reduces them.
      int splits = 1;
      KMD_HIP(c, kmd::gemm_partials<T>("gemm_out:splitk", attn, D, (const T *)lw.oW, D, M, D, D, sk, &splits, s));
      if (splits > 1) {
        KMD_HIP(c, kmd::add_layernorm_splitk<T>(h, sk.partial, splits, lw.ob, lw.ln1g, lw.ln1b, h1, M, s));
      } else {
        KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_OUT, attn, D, (const T *)lw.oW, D, lw.ob, tmp, D, M, D, D, s));
        KMD_HIP(c, kmd::add_layernorm<T>(h, tmp, lw.ln1g, lw.ln1b, h1, M, s));
      }
      KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_FFN1, h1, D, (const T *)lw.ff1W, D, lw.ff1b, ffn, F, M, F, D, s, sk));
      KMD_HIP(c, kmd::gemm_partials<T>("gemm_ffn2:splitk", ffn, F, (const T *)lw.ff2W, F, M, D, F, sk, &splits, s));
      if (splits > 1) {
        KMD_HIP(c, kmd::add_layernorm_splitk<T>(h1, sk.partial, splits, lw.ff2b, lw.ln2g, lw.ln2b, h, M, s));
      } else {
        KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_FFN2, ffn, F, (const T *)lw.ff2W, F, lw.ff2b, tmp, D, M, D, F, s));
        KMD_HIP(c, kmd::add_layernorm<T>(h1, tmp, lw.ln2g, lw.ln2b, h, M, s));
      }
      if (tr && tr->layers)  // dense [2B][T + 2][1024] copy, padded tokens 0
        KMD_HIP(c, kmd::unpack_rows(h, D * (int)sizeof(T), tok, mot, P, 0, S,
                                    static_cast<char *>(tr->layers) + layer_index * all_rows_bytes +
                                        rt * D * sizeof(T),
                                    s));
      ++layer_index;
    }
    KMD_HIP(c, kmd::gemm<T>(kmd::ROLE_HEAD, h, D, (const T *)nw.outW, D, nw.outb, head[n], nw.n_out, M, nw.n_out, D,
                            s, sk));
    float *dst = tr ? (n == 0 ? tr->root_out : tr->body_out) : nullptr;
    if (dst)  // the motion rows, dense [P][T][n_out], padded frames 0
      KMD_HIP(c, kmd::unpack_rows(head[n], nw.n_out * (int)sizeof(float), tok, mot, P, 2, T_, dst + f0 * nw.n_out,
                                  s));
  }
  return KIMODO_OK;
}

// Whether a step runs both guidance groups as one chain of 2B sequences
// rather than as two concurrent chains of B, from the clips' packed token rows.
// Eager steps and captured graphs decide alike, so they stay bitwise equal.
inline bool merge_groups(const std::vector<int32_t> &len) {
  int64_t rows = 0;
  for (int32_t l : len) rows += 2 * ((l + 2 + 7) & ~7);
  return rows <= MERGE_MAX_ROWS;
}

// One DDIM step of B clips: reads x_t, writes x_prev (may alias), per-step
// scalars at the device step counter, which it decrements at the end. known /
// kmask: the clips' known entries ([B][T][279]) or both null.
// concurrent: chain j > 0 runs on its own stream, forked from and joined back
// to s, so the chains' kernels overlap (in the captured graph and in the
// profiled step); otherwise the chains run one after the other on s, with the
// same arithmetic.
template <typename T>
kimodo_status enqueue_step(kimodo_ctx *c, int B, int T_, const float *x_t, float *x_prev, float w,
                           const float *known, const uint8_t *kmask, const kimodo_trace *tr, hipStream_t s,
                           bool concurrent = false) {
  const Layout &L = c->L;
  // one chain over both guidance groups, or one chain per group
  const bool merged = merge_groups(c->h_len);
  const int chains = merged ? 1 : MAX_CHAINS;
  concurrent = concurrent && chains > 1;
  if (concurrent) {
    KMD_HIP(c, hipEventRecord(c->fork_event, s));
    for (int j = 1; j < chains; ++j) KMD_HIP(c, hipStreamWaitEvent(c->chain_stream[j - 1], c->fork_event, 0));
  }
  kimodo_status st = KIMODO_OK;
  for (int j = 0; j < chains && st == KIMODO_OK; ++j)
    st = enqueue_group<T>(c, B, T_, j, 0, B, merged ? 2 : 1, x_t, known, kmask, tr,
                          concurrent && j > 0 ? c->chain_stream[j - 1] : s);
  if (concurrent) {
    for (int j = 1; j < chains; ++j) {
      KMD_HIP(c, hipEventRecord(c->join_event[j - 1], c->chain_stream[j - 1]));
      KMD_HIP(c, hipStreamWaitEvent(s, c->join_event[j - 1], 0));
    }
  }
  if (st != KIMODO_OK) return st;
  int32_t *counter = c->at<int32_t>(L.counter);
  KMD_HIP(c, kmd::cfg_ddim(c->at<float>(L.head_root), c->at<float>(L.head_body), x_t, x_prev, c->at<float>(L.coef),
                           counter, c->at<int32_t>(L.lengths), c->at<int32_t>(L.tok_g), known, kmask, B, T_, w,
                           tr ? tr->x0_hat : nullptr, s));
  KMD_HIP(c, kmd::step_advance(counter, s));
  return KIMODO_OK;
}

// DDIM (eta = 0) as x_prev = c_x0 x0_hat + c_xt x_t with coefficients in fp64:
// c_xt = sqrt(1 - ab_prev) / sqrt(1 - ab_t), c_x0 = sqrt(ab_prev) - c_xt sqrt(ab_t).
void ddim_coef(double ab_t, double ab_prev, float *out) {
  const double cxt = std::sqrt(1.0 - ab_prev) / std::sqrt(1.0 - ab_t);
  out[0] = (float)(std::sqrt(ab_prev) - cxt * std::sqrt(ab_t));
  out[1] = (float)cxt;
}

// Uploads lengths, timesteps and DDIM coefficients (k = 0..S-1), sets the
// step counter to S - 1, and builds the token-row packing of the step's
// chains: sequence q of a chain (clip q % B) has lengths[q % B] + 2 token rows,
// packed without the padded frames.
kimodo_status upload_tables(kimodo_ctx *c, int B, int T_, const int32_t *lengths, const int32_t *timesteps,
                            const double *abar, double abar_prev0, int S, hipStream_t s) {
  c->h_steps.assign(timesteps, timesteps + S);
  c->h_coef.resize(2 * S);
  for (int k = 0; k < S; ++k) ddim_coef(abar[k], k > 0 ? abar[k - 1] : abar_prev0, &c->h_coef[2 * k]);
  if (lengths)
    c->h_len.assign(lengths, lengths + B);
  else
    c->h_len.assign(B, T_);
  KMD_HIP(c, hipMemcpyAsync(c->at<int32_t>(c->L.lengths), c->h_len.data(), sizeof(int32_t) * B,
                            hipMemcpyHostToDevice, s));
  const int Pc = merge_groups(c->h_len) ? 2 * B : B;  // sequences per chain
  c->h_tok.resize(Pc + 1);
  c->h_mot.resize(Pc + 1);
  int tok = 0, mot = 0;
  for (int q = 0; q < Pc; ++q) {
    c->h_tok[q] = tok;
    c->h_mot[q] = mot;
    const int len = c->h_len[q % B];
    tok += (len + 2 + 7) & ~7;
    mot += len;
  }
  c->h_tok[Pc] = tok;
  c->h_mot[Pc] = mot;
  c->m_tok = tok;
  c->m_mot = mot;
  // sequence p's token rows in the whole activation buffers: chain j of two
  // starts at row j B seq_rows(T)
  c->h_tok_g.resize(2 * B);
  for (int p = 0; p < 2 * B; ++p)
    c->h_tok_g[p] = Pc == 2 * B ? c->h_tok[p] : (p / B) * B * seq_rows(T_) + c->h_tok[p % B];
  KMD_HIP(c, hipMemcpyAsync(c->at<int32_t>(c->L.tok), c->h_tok.data(), sizeof(int32_t) * (Pc + 1),
                            hipMemcpyHostToDevice, s));
  KMD_HIP(c, hipMemcpyAsync(c->at<int32_t>(c->L.mot), c->h_mot.data(), sizeof(int32_t) * (Pc + 1),
                            hipMemcpyHostToDevice, s));
  KMD_HIP(c, hipMemcpyAsync(c->at<int32_t>(c->L.tok_g), c->h_tok_g.data(), sizeof(int32_t) * 2 * B,
                            hipMemcpyHostToDevice, s));
  KMD_HIP(c, kmd::packing_maps(c->at<int32_t>(c->L.tok), Pc, seq_rows(T_), c->at<int32_t>(c->L.row_ps), s));
  KMD_HIP(c, hipMemcpyAsync(c->at<int32_t>(c->L.steps), c->h_steps.data(), sizeof(int32_t) * S,
                            hipMemcpyHostToDevice, s));
  KMD_HIP(c, hipMemcpyAsync(c->at<float>(c->L.coef), c->h_coef.data(), sizeof(float) * 2 * S, hipMemcpyHostToDevice,
                            s));
  KMD_HIP(c, kmd::set_int(c->at<int32_t>(c->L.counter), S - 1, s));
  return KIMODO_OK;
}

kimodo_status check_call(kimodo_ctx *c, int B, int T_, const float *x, const float *text, const int32_t *lengths,
                         float w, const float *out) {
  if (!c) return KIMODO_ESTATE;
  c->err.clear();
  if (!x || !text || !out) return fail(c, KIMODO_EINVAL, "null tensor pointer");
  if (B < 1 || B > c->cfg.max_batch) return fail(c, KIMODO_ESHAPE, "B out of 1..max_batch");
  if (T_ < 1 || T_ > c->cfg.max_frames) return fail(c, KIMODO_ESHAPE, "T out of 1..max_frames");
  if (!std::isfinite(w)) return fail(c, KIMODO_EINVAL, "cfg_scale is not finite");
  if (lengths)
    for (int b = 0; b < B; ++b)
      if (lengths[b] < 1 || lengths[b] > T_) return fail(c, KIMODO_ESHAPE, "lengths[b] out of 1..T");
  return KIMODO_OK;
}

template <typename T>
// concurrent: the guidance groups on two streams, as in the captured graph
// (the profiled step); otherwise one after the other on s.
kimodo_status denoise_step_t(kimodo_ctx *c, int B, int T_, const float *x_t, const float *text,
                             const int32_t *lengths, int32_t t, double ab_t, double ab_prev, float w,
                             const float *known, const uint8_t *kmask, float *x_prev, const kimodo_trace *tr,
                             hipStream_t s, bool concurrent = false) {
  kimodo_status st = init_device<T>(c, s);
  if (st == KIMODO_OK) st = upload_tables(c, B, T_, lengths, &t, &ab_t, ab_prev, 1, s);
  if (st == KIMODO_OK) st = conditioning_tokens<T>(c, B, text, 1, s);
  if (st == KIMODO_OK) st = enqueue_step<T>(c, B, T_, x_t, x_prev, w, known, kmask, tr, s, concurrent);
  return st;
}

// The step graph reads the state, and with constrained set the known entries,
// from fixed workspace buffers. Graphs are cached by (B, T, w, constrained,
// lengths) (the lengths fix the packed row counts, i.e. the grid sizes, of its
// launches). A miss reuses a slot of the same (B, T, w, constrained) if there
// is one, else the least recently used slot; when the new capture has the same
// kernels as that slot's graph (the usual case when only lengths change), the
// executable graph is updated in place instead of instantiated again, which is
// several times cheaper. upload_tables has run for this call.
template <typename T>
kimodo_status capture_step(kimodo_ctx *c, int B, int T_, float w, bool constrained, StepGraph **out) {
  StepGraph *slot = &c->graphs[0], *sibling = nullptr;
  for (StepGraph &g : c->graphs) {
    const bool same_shape = g.exec && g.B == B && g.T == T_ && g.w == w && g.constrained == constrained;
    if (same_shape && g.len == c->h_len) {
      g.last_use = ++c->graph_clock;
      *out = &g;
      return KIMODO_OK;
    }
    if (same_shape && (!sibling || g.last_use < sibling->last_use)) sibling = &g;
    if (!g.exec || (slot->exec && g.last_use < slot->last_use)) slot = &g;
  }
  if (sibling) slot = sibling;
  // replays of the replaced or updated graph may still be queued on the caller's stream
  if (slot->done_recorded) KMD_HIP(c, hipEventSynchronize(slot->done));
  slot->done_recorded = false;
  float *state = c->at<float>(c->L.state);
  const float *known = constrained ? c->at<float>(c->L.known) : nullptr;
  const uint8_t *kmask = constrained ? c->at<uint8_t>(c->L.kmask) : nullptr;
  KMD_HIP(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
  kimodo_status st = enqueue_step<T>(c, B, T_, state, state, w, known, kmask, nullptr, c->cap_stream, true);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(c->cap_stream, &g);
  if (st != KIMODO_OK) {
    if (g) (void)hipGraphDestroy(g);
    return st;
  }
  if (e != hipSuccess) return fail(c, KIMODO_EHIP, std::string("graph capture: ") + hipGetErrorString(e));
  bool updated = false;
  if (slot == sibling) {
    hipGraphNode_t bad = nullptr;
    hipGraphExecUpdateResult res = hipGraphExecUpdateError;
    updated = hipGraphExecUpdate(slot->exec, g, &bad, &res) == hipSuccess && res == hipGraphExecUpdateSuccess;
    if (!updated) (void)hipGetLastError();  // a refused update leaves the old executable graph as it was
  }
  if (updated) {
    ++c->graph_updates;
  } else {
    if (slot->exec) KMD_HIP(c, hipGraphExecDestroy(slot->exec));
    slot->exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&slot->exec, g, nullptr, nullptr, 0);
    if (ei != hipSuccess) {
      slot->exec = nullptr;
      if (slot->graph) (void)hipGraphDestroy(slot->graph);
      slot->graph = nullptr;
      slot->B = -1;
      (void)hipGraphDestroy(g);
      return fail(c, KIMODO_EHIP, std::string("graph instantiate: ") + hipGetErrorString(ei));
    }
    ++c->graph_instantiations;
  }
  if (slot->graph) KMD_HIP(c, hipGraphDestroy(slot->graph));
  slot->graph = g;
  slot->B = B;
  slot->T = T_;
  slot->w = w;
  slot->len = c->h_len;
  slot->constrained = constrained;
  slot->last_use = ++c->graph_clock;
  *out = slot;
  return KIMODO_OK;
}

// The S-step loop from noise, leaving x_0 in the workspace state buffer. With
// constrained set, the known entries are read from the workspace known / kmask
// buffers, which the caller has filled in stream order.
template <typename T>
kimodo_status run_sample(kimodo_ctx *c, int B, int T_, const float *noise, const float *text, const int32_t *lengths,
                         const int32_t *timesteps, const double *abar, int S, float w, bool constrained,
                         hipStream_t s) {
  kimodo_status st = init_device<T>(c, s);
  if (st == KIMODO_OK) st = upload_tables(c, B, T_, lengths, timesteps, abar, 1.0, S, s);
  if (st == KIMODO_OK) st = conditioning_tokens<T>(c, B, text, S, s);
  StepGraph *g = nullptr;
  if (st == KIMODO_OK) st = capture_step<T>(c, B, T_, w, constrained, &g);
  if (st != KIMODO_OK) return st;
  float *state = c->at<float>(c->L.state);
  KMD_HIP(c, hipMemcpyAsync(state, noise, (size_t)B * T_ * FEATS * sizeof(float), hipMemcpyDeviceToDevice, s));
  for (int k = 0; k < S; ++k) KMD_HIP(c, hipGraphLaunch(g->exec, s));
  KMD_HIP(c, hipEventRecord(g->done, s));
  g->done_recorded = true;
  return KIMODO_OK;
}

template <typename T>
kimodo_status sample_t(kimodo_ctx *c, int B, int T_, const float *noise, const float *text, const int32_t *lengths,
                       const int32_t *timesteps, const double *abar, int S, float w, const float *known,
                       const uint8_t *kmask, float *out, hipStream_t s) {
  const size_t n = (size_t)B * T_ * FEATS;
  if (known) {
    KMD_HIP(c, hipMemcpyAsync(c->at<float>(c->L.known), known, n * sizeof(float), hipMemcpyDeviceToDevice, s));
    KMD_HIP(c, hipMemcpyAsync(c->at<uint8_t>(c->L.kmask), kmask, n, hipMemcpyDeviceToDevice, s));
  }
  kimodo_status st = run_sample<T>(c, B, T_, noise, text, lengths, timesteps, abar, S, w, known != nullptr, s);
  if (st != KIMODO_OK) return st;
  KMD_HIP(c, hipMemcpyAsync(out, c->at<float>(c->L.state), n * sizeof(float), hipMemcpyDeviceToDevice, s));
  return KIMODO_OK;
}

// Segments one after another on s. Segment k covers timeline frames start_k ..
// start_k + T_k - 1 with start_k = start_{k-1} + T_{k-1} - n_tr; its first n_tr
// frames are known and equal to the last n_tr frames of segment k-1, which are
// already in out at start_k .., and it writes frames start_k + n_tr .. to out.
template <typename T>
kimodo_status timeline_t(kimodo_ctx *c, int V, int n_seg, const int32_t *seg_frames, const float *seg_text,
                         const float *noise, int n_tr, const int32_t *timesteps, const double *abar, int S, float w,
                         float *out, int total, hipStream_t s) {
  const float *state = c->at<float>(c->L.state);
  size_t noise_off = 0;
  int start = 0;
  for (int k = 0; k < n_seg; ++k) {
    const int Tk = seg_frames[k];
    const bool constrained = k > 0 && n_tr > 0;
    if (constrained)
      KMD_HIP(c, kmd::tail_known(out, total, start, V, Tk, n_tr, c->at<float>(c->L.known),
                                 c->at<uint8_t>(c->L.kmask), s));
    kimodo_status st = run_sample<T>(c, V, Tk, noise + noise_off, seg_text + (size_t)k * V * TEXT, nullptr,
                                     timesteps, abar, S, w, constrained, s);
    if (st != KIMODO_OK) return st;
    const int skip = k > 0 ? n_tr : 0;
    KMD_HIP(c, hipMemcpy2DAsync(out + ((size_t)start + skip) * FEATS, (size_t)total * FEATS * sizeof(float),
                                state + (size_t)skip * FEATS, (size_t)Tk * FEATS * sizeof(float),
                                (size_t)(Tk - skip) * FEATS * sizeof(float), V, hipMemcpyDeviceToDevice, s));
    noise_off += (size_t)V * Tk * FEATS;
    if (k + 1 < n_seg) start += Tk - n_tr;
  }
  return KIMODO_OK;
}

// Hands out start/stop event pairs from the ctx's pool, one per launch.
struct EventTimer : kmd::KernelTimer {
  std::vector<hipEvent_t> *pool;
  std::vector<std::string> names;
  hipError_t err = hipSuccess;
  bool slot(const char *name, hipEvent_t *start, hipEvent_t *stop) override {
    const size_t i = names.size();
    while (pool->size() < 2 * (i + 1)) {
      hipEvent_t e;
      if ((err = hipEventCreate(&e)) != hipSuccess) return false;
      pool->push_back(e);
    }
    *start = (*pool)[2 * i];
    *stop = (*pool)[2 * i + 1];
    names.emplace_back(name);
    return true;
  }
};

struct TimerScope {
  explicit TimerScope(kmd::KernelTimer *t) { kmd::kernel_timer() = t; }
  ~TimerScope() { kmd::kernel_timer() = nullptr; }
};

kimodo_status check_schedule(kimodo_ctx *ctx, const int32_t *timesteps, const double *abar, int S) {
  if (!timesteps || !abar) return fail(ctx, KIMODO_EINVAL, "null timesteps or abar");
  if (S < 1 || S > ctx->cfg.max_steps) return fail(ctx, KIMODO_ESHAPE, "S out of 1..max_steps");
  for (int k = 0; k < S; ++k) {
    if (timesteps[k] < 0 || timesteps[k] >= 100000 || (k > 0 && timesteps[k] <= timesteps[k - 1]))
      return fail(ctx, KIMODO_ESHAPE, "timesteps must be strictly ascending in 0..99999");
    if (!(abar[k] > 0.0 && abar[k] < 1.0)) return fail(ctx, KIMODO_EINVAL, "abar[k] not in (0, 1)");
  }
  return KIMODO_OK;
}

kimodo_status check_known(kimodo_ctx *ctx, const float *known, const uint8_t *kmask) {
  if ((known == nullptr) != (kmask == nullptr))
    return fail(ctx, KIMODO_EINVAL, "known_values and known_mask must both be set or both be NULL");
  if (known && (reinterpret_cast<uintptr_t>(known) & 3)) return fail(ctx, KIMODO_EINVAL, "known_values misaligned");
  return KIMODO_OK;
}

kimodo_status check_step(kimodo_ctx *ctx, int B, int T, const float *x_t, const float *text, const int32_t *lengths,
                         int32_t t, double abar_t, double abar_prev, float w, const float *x_prev) {
  kimodo_status st = check_call(ctx, B, T, x_t, text, lengths, w, x_prev);
  if (st != KIMODO_OK) return st;
  if (t < 0 || t >= 100000) return fail(ctx, KIMODO_ESHAPE, "t out of 0..99999");
  if (!(abar_t > 0.0 && abar_t < 1.0)) return fail(ctx, KIMODO_EINVAL, "abar_t not in (0, 1)");
  if (!(abar_prev > 0.0 && abar_prev <= 1.0)) return fail(ctx, KIMODO_EINVAL, "abar_prev not in (0, 1]");
  return KIMODO_OK;
}

template <typename T>
kimodo_status profile_step_t(kimodo_ctx *c, int B, int T_, const float *x_t, const float *text,
                             const int32_t *lengths, int32_t t, double ab_t, double ab_prev, float w, float *x_prev,
                             kimodo_kernel_time *records, int max_records, int32_t *n_records, hipStream_t s) {
  kimodo_status st = init_device<T>(c, s);
  if (st != KIMODO_OK) return st;
  EventTimer timer;
  timer.pool = &c->events;
  {
    TimerScope scope(&timer);
    // the chains one after the other: each kernel has the GPU to itself, so its
    // events time it alone (as a kernel trace does)
    st = denoise_step_t<T>(c, B, T_, x_t, text, lengths, t, ab_t, ab_prev, w, nullptr, nullptr, x_prev, nullptr, s,
                           false);
  }
  if (timer.err != hipSuccess) return fail(c, KIMODO_EHIP, std::string("hipEventCreate: ") + hipGetErrorString(timer.err));
  if (st != KIMODO_OK) return st;
  KMD_HIP(c, hipStreamSynchronize(s));
  const int n = (int)timer.names.size();
  for (int i = 0; i < n && i < max_records; ++i) {
    float ms = 0.f;
    KMD_HIP(c, hipEventElapsedTime(&ms, c->events[2 * i], c->events[2 * i + 1]));
    std::memset(records[i].name, 0, sizeof(records[i].name));
    std::strncpy(records[i].name, timer.names[i].c_str(), sizeof(records[i].name) - 1);
    records[i].ms = ms;
  }
  *n_records = n;
  return KIMODO_OK;
}

// Points c at its workspace and layout, and maps the canonical weight table
// onto the network structs: tensors the kernels read as they are, or their
// converted copies in the workspace (with the set-up pass of each listed in
// c->conversions).
void bind(kimodo_ctx *c, const kimodo_config &cfg, const void *const *weights, char *ws, const Layout &L) {
  c->cfg = cfg;
  c->ws = ws;
  c->L = L;
  c->conversions.clear();
  const WeightPlan wp = plan_weights(cfg);
  const int n_weights = weight_count(cfg);
  std::vector<const void *> dev(n_weights);
  for (int i = 0; i < n_weights; ++i) {
    if (wp.off[i] == SIZE_MAX) {
      dev[i] = weights[i];
      c->conversions.push_back({weights[i], nullptr, wp.n[i], false});
    } else {
      void *dst = c->ws + L.weights + wp.off[i];
      c->conversions.push_back({weights[i], dst, wp.n[i], wp.matrix[i]});
      dev[i] = dst;
    }
  }
  int idx = 0;
  auto mat = [&]() { return dev[idx++]; };
  auto vec = [&]() { return static_cast<const float *>(dev[idx++]); };
  for (int n = 0; n < 2; ++n) {
    NetW &w = c->net[n];
    w.layers.clear();
    w.txtW = mat();
    w.txtb = vec();
    w.t1W = mat();
    w.t1b = vec();
    w.t2W = mat();
    w.t2b = vec();
    w.inW = mat();
    w.inb = vec();
    const int nl = n ? cfg.layers_body : cfg.layers_root;
    for (int l = 0; l < nl; ++l) {
      LayerW lw;
      lw.qkvW = mat();
      lw.qkvb = vec();
      lw.oW = mat();
      lw.ob = vec();
      lw.ln1g = vec();
      lw.ln1b = vec();
      lw.ff1W = mat();
      lw.ff1b = vec();
      lw.ff2W = mat();
      lw.ff2b = vec();
      lw.ln2g = vec();
      lw.ln2b = vec();
      w.layers.push_back(lw);
    }
    w.outW = mat();
    w.outb = vec();
    w.k_in = n ? FEATS : ROOT;
    w.kpad = n ? KPAD_BODY : KPAD_ROOT;
    w.n_out = n ? BODY : ROOT;
    w.in_pad = c->ws + L.in_pad[n];
  }
}

}  // namespace

// Scratch of kimodo_denoise_step_static, the one entry point that allocates
// nothing: the whole workspace of its step (activations, split-K partial sums,
// tables, converted weight vectors). Each GPU the library runs on holds its
// own copy until the process ends. In host code the name is only a stand-in:
// kernels are given the device address that scratch_address looks up.
constexpr size_t STATIC_SCRATCH_BYTES = size_t(96) << 20;
static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void *scratch_device[MAX_DEVICES] = {};

// Device address of the current GPU's copy of scratch, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_device[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_device[dev] = p;
  }
  *out = scratch_device[dev];
  return hipSuccess;
}

// kimodo_denoise_step's work for a ctx whose workspace is the scratch array:
// the set-up of weights and tables runs on every call (the array keeps
// whatever the last call left), with no host wait.
template <typename T>
kimodo_status static_step_t(kimodo_ctx *c, int B, int T_, const float *x_t, const float *text,
                            const int32_t *lengths, int32_t t, double ab_t, double ab_prev, float w, float *x_prev,
                            hipStream_t s) {
  kimodo_status st = setup_tables<T>(c, s);
  if (st == KIMODO_OK) st = upload_tables(c, B, T_, lengths, &t, &ab_t, ab_prev, 1, s);
  if (st == KIMODO_OK) st = conditioning_tokens<T>(c, B, text, 1, s);
  if (st == KIMODO_OK) st = enqueue_step<T>(c, B, T_, x_t, x_prev, w, nullptr, nullptr, nullptr, s, false);
  return st;
}

}  // namespace

namespace kmd {
KernelTimer *&kernel_timer() {
  static thread_local KernelTimer *t = nullptr;
  return t;
}
}  // namespace kmd

extern "C" {

size_t kimodo_workspace_bytes(const kimodo_config *cfg) { return config_ok(cfg) ? plan(*cfg).total : 0; }

int32_t kimodo_weight_count(const kimodo_config *cfg) { return config_ok(cfg) ? weight_count(*cfg) : -1; }

kimodo_status kimodo_weight_shape(const kimodo_config *cfg, int32_t index, int32_t *ndim, int64_t shape[2]) {
  if (!config_ok(cfg)) return KIMODO_ECONFIG;
  if (!ndim || !shape) return KIMODO_EINVAL;
  if (index < 0 || index >= weight_count(*cfg)) return KIMODO_EINVAL;
  weight_shape(*cfg, index, &shape[0], &shape[1]);
  *ndim = shape[1] ? 2 : 1;
  return KIMODO_OK;
}

kimodo_status kimodo_make_schedule(int32_t n_train, double beta_start, double beta_end, int32_t S,
                                   int32_t *timesteps, double *abar) {
  if (!timesteps || !abar) return KIMODO_EINVAL;
  if (n_train < 2 || n_train > 100000 || S < 1 || S > n_train) return KIMODO_ESHAPE;
  if (!(beta_start > 0.0) || !(beta_end >= beta_start) || !(beta_end < 1.0)) return KIMODO_EINVAL;
  std::vector<double> ab(n_train);
  double prod = 1.0;
  for (int i = 0; i < n_train; ++i) {
    prod *= 1.0 - (beta_start + (beta_end - beta_start) * (double)i / (double)(n_train - 1));
    ab[i] = prod;
  }
  for (int k = 0; k < S; ++k) {
    const int t = (int)(((int64_t)k * n_train) / S);
    timesteps[k] = t;
    abar[k] = ab[t];
  }
  return KIMODO_OK;
}

kimodo_status kimodo_make_cosine_schedule(int32_t n_train, double s, double max_beta, int32_t S,
                                          int32_t *timesteps, double *abar) {
  if (!timesteps || !abar) return KIMODO_EINVAL;
  if (n_train < 2 || n_train > 100000 || S < 1 || S > n_train) return KIMODO_ESHAPE;
  if (!(s >= 0.0 && s <= 1.0) || !(max_beta > 0.0 && max_beta < 1.0)) return KIMODO_EINVAL;
  // f(u) = cos^2(pi/2 (u + s) / (1 + s)); beta_i from consecutive ratios, clipped.
  const double half_pi = 1.5707963267948966;
  auto f = [&](double u) {
    const double c = std::cos(half_pi * (u + s) / (1.0 + s));
    return c * c;
  };
  std::vector<double> ab(n_train);
  double prod = 1.0;
  for (int i = 0; i < n_train; ++i) {
    const double beta = std::min(1.0 - f((double)(i + 1) / n_train) / f((double)i / n_train), max_beta);
    prod *= 1.0 - beta;
    ab[i] = prod;
  }
  for (int k = 0; k < S; ++k) {
    const int t = (int)(((int64_t)k * n_train) / S);
    timesteps[k] = t;
    abar[k] = ab[t];
  }
  return KIMODO_OK;
}

kimodo_status kimodo_create(const kimodo_config *cfg, const void *const *weights, int32_t n_weights,
                            void *workspace, size_t workspace_bytes, kimodo_stream stream, kimodo_ctx **out) {
  (void)stream;
  if (!out) return KIMODO_EINVAL;
  *out = nullptr;
  if (!cfg) return KIMODO_EINVAL;
  if (!config_ok(cfg))
    return (cfg->dtype < KIMODO_F32 || cfg->dtype > KIMODO_F16) ? KIMODO_EDTYPE : KIMODO_ECONFIG;
  if (!weights || n_weights != weight_count(*cfg)) return KIMODO_EWEIGHTS;
  for (int i = 0; i < n_weights; ++i)
    if (!weights[i] || (reinterpret_cast<uintptr_t>(weights[i]) & 15)) return KIMODO_EWEIGHTS;
  const Layout L = plan(*cfg);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) || workspace_bytes < L.total)
    return KIMODO_EWORKSPACE;
  kimodo_ctx *c = new (std::nothrow) kimodo_ctx();
  if (!c) return KIMODO_ESTATE;
  bind(c, *cfg, weights, static_cast<char *>(workspace), L);
  *out = c;
  return KIMODO_OK;
}

kimodo_status kimodo_denoise_step_constrained(kimodo_ctx *ctx, int32_t B, int32_t T, const float *x_t,
                                              const float *text_emb, const int32_t *lengths, int32_t t,
                                              double abar_t, double abar_prev, float cfg_scale,
                                              const float *known_values, const uint8_t *known_mask, float *x_prev,
                                              const kimodo_trace *trace, kimodo_stream stream) {
  kimodo_status st = check_step(ctx, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, x_prev);
  if (st != KIMODO_OK) return st;
  if ((st = check_known(ctx, known_values, known_mask)) != KIMODO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ctx->cfg.dtype == KIMODO_F32)
    return denoise_step_t<float>(ctx, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, known_values,
                                 known_mask, x_prev, trace, s);
  return denoise_step_t<f16>(ctx, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, known_values,
                             known_mask, x_prev, trace, s);
}

kimodo_status kimodo_denoise_step(kimodo_ctx *ctx, int32_t B, int32_t T, const float *x_t, const float *text_emb,
                                  const int32_t *lengths, int32_t t, double abar_t, double abar_prev,
                                  float cfg_scale, float *x_prev, const kimodo_trace *trace, kimodo_stream stream) {
  return kimodo_denoise_step_constrained(ctx, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, nullptr,
                                         nullptr, x_prev, trace, stream);
}

kimodo_status kimodo_denoise_step_static(const kimodo_config *cfg, const void *const *weights, int32_t n_weights,
                                         int32_t B, int32_t T, const float *x_t, const float *text_emb,
                                         const int32_t *lengths, int32_t t, double abar_t, double abar_prev,
                                         float cfg_scale, float *x_prev, kimodo_stream stream) {
  if (!cfg) return KIMODO_EINVAL;
  if (cfg->dtype != KIMODO_F32 && cfg->dtype != KIMODO_F16) return KIMODO_EDTYPE;
  kimodo_config call = *cfg;  // a workspace sized for exactly this call
  call.max_batch = B;
  call.max_frames = T;
  call.max_steps = 1;
  if (B < 1 || B > 512 || T < 1 || T > 4096) return KIMODO_ESHAPE;
  if (!config_ok(&call)) return KIMODO_ECONFIG;
  if (!weights || n_weights != weight_count(call)) return KIMODO_EWEIGHTS;
  for (int i = 0; i < n_weights; ++i)
    if (!weights[i] || (reinterpret_cast<uintptr_t>(weights[i]) & 15)) return KIMODO_EWEIGHTS;
  const Layout L = plan(call);
  if (L.total > STATIC_SCRATCH_BYTES) return KIMODO_EWORKSPACE;
  // host-side state of the call (tables staged for upload), kept per thread
  // until its next call
  thread_local kimodo_ctx c;
  c.cfg = call;
  kimodo_status st = check_step(&c, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, x_prev);
  if (st != KIMODO_OK) return st;
  void *base = nullptr;
  if (scratch_address(&base) != hipSuccess) return KIMODO_EHIP;
  bind(&c, call, weights, static_cast<char *>(base), L);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (call.dtype == KIMODO_F32)
    return static_step_t<float>(&c, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, x_prev, s);
  return static_step_t<f16>(&c, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, x_prev, s);
}

kimodo_status kimodo_sample_constrained(kimodo_ctx *ctx, int32_t B, int32_t T, const float *noise,
                                        const float *text_emb, const int32_t *lengths, const int32_t *timesteps,
                                        const double *abar, int32_t S, float cfg_scale, const float *known_values,
                                        const uint8_t *known_mask, float *out, kimodo_stream stream) {
  kimodo_status st = check_call(ctx, B, T, noise, text_emb, lengths, cfg_scale, out);
  if (st != KIMODO_OK) return st;
  if ((st = check_schedule(ctx, timesteps, abar, S)) != KIMODO_OK) return st;
  if ((st = check_known(ctx, known_values, known_mask)) != KIMODO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ctx->cfg.dtype == KIMODO_F32)
    return sample_t<float>(ctx, B, T, noise, text_emb, lengths, timesteps, abar, S, cfg_scale, known_values,
                           known_mask, out, s);
  return sample_t<f16>(ctx, B, T, noise, text_emb, lengths, timesteps, abar, S, cfg_scale, known_values, known_mask,
                       out, s);
}

kimodo_status kimodo_sample(kimodo_ctx *ctx, int32_t B, int32_t T, const float *noise, const float *text_emb,
                            const int32_t *lengths, const int32_t *timesteps, const double *abar, int32_t S,
                            float cfg_scale, float *out, kimodo_stream stream) {
  return kimodo_sample_constrained(ctx, B, T, noise, text_emb, lengths, timesteps, abar, S, cfg_scale, nullptr,
                                   nullptr, out, stream);
}

kimodo_status kimodo_sample_timeline(kimodo_ctx *ctx, int32_t V, int32_t n_seg, const int32_t *seg_frames,
                                     const float *seg_text, const float *noise, int32_t n_transition,
                                     const int32_t *timesteps, const double *abar, int32_t S, float cfg_scale,
                                     float *out, kimodo_stream stream) {
  if (!ctx) return KIMODO_ESTATE;
  ctx->err.clear();
  if (!seg_frames || !seg_text || !noise || !out) return fail(ctx, KIMODO_EINVAL, "null pointer argument");
  if (V < 1 || V > ctx->cfg.max_batch) return fail(ctx, KIMODO_ESHAPE, "V out of 1..max_batch");
  if (n_seg < 1 || n_seg > 1024) return fail(ctx, KIMODO_ESHAPE, "n_seg out of 1..1024");
  if (!std::isfinite(cfg_scale)) return fail(ctx, KIMODO_EINVAL, "cfg_scale is not finite");
  if (n_transition < 0) return fail(ctx, KIMODO_ESHAPE, "n_transition < 0");
  int64_t total = 0;
  for (int k = 0; k < n_seg; ++k) {
    const int Tk = seg_frames[k];
    if (Tk < 1 || Tk > ctx->cfg.max_frames) return fail(ctx, KIMODO_ESHAPE, "seg_frames[k] out of 1..max_frames");
    if (k > 0 && (n_transition >= Tk || n_transition > seg_frames[k - 1]))
      return fail(ctx, KIMODO_ESHAPE, "n_transition must be < T_k and <= T_{k-1}");
    total += k > 0 ? Tk - n_transition : Tk;
  }
  if (total > INT32_MAX / FEATS) return fail(ctx, KIMODO_ESHAPE, "timeline too long");
  kimodo_status st = check_schedule(ctx, timesteps, abar, S);
  if (st != KIMODO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ctx->cfg.dtype == KIMODO_F32)
    return timeline_t<float>(ctx, V, n_seg, seg_frames, seg_text, noise, n_transition, timesteps, abar, S, cfg_scale,
                             out, (int)total, s);
  return timeline_t<f16>(ctx, V, n_seg, seg_frames, seg_text, noise, n_transition, timesteps, abar, S, cfg_scale, out,
                         (int)total, s);
}

kimodo_status kimodo_profile_step(kimodo_ctx *ctx, int32_t B, int32_t T, const float *x_t, const float *text_emb,
                                  const int32_t *lengths, int32_t t, double abar_t, double abar_prev,
                                  float cfg_scale, float *x_prev, kimodo_kernel_time *records, int32_t max_records,
                                  int32_t *n_records, kimodo_stream stream) {
  kimodo_status st = check_step(ctx, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, x_prev);
  if (st != KIMODO_OK) return st;
  if (!n_records || max_records < 0 || (max_records > 0 && !records))
    return fail(ctx, KIMODO_EINVAL, "records / n_records");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ctx->cfg.dtype == KIMODO_F32)
    return profile_step_t<float>(ctx, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, x_prev, records,
                                 max_records, n_records, s);
  return profile_step_t<f16>(ctx, B, T, x_t, text_emb, lengths, t, abar_t, abar_prev, cfg_scale, x_prev, records,
                             max_records, n_records, s);
}

kimodo_status kimodo_fk(int32_t n_frames, const float *motion, const int32_t *parents, const float *offsets,
                        float *positions, float *rotations, kimodo_stream stream) {
  if (n_frames < 0 || n_frames > (1 << 26)) return KIMODO_ESHAPE;
  if (!motion || !parents || !offsets || !positions) return KIMODO_EINVAL;
  if ((reinterpret_cast<uintptr_t>(motion) | reinterpret_cast<uintptr_t>(positions) |
       reinterpret_cast<uintptr_t>(rotations)) & 3)
    return KIMODO_EINVAL;
  kmd::FkSkeleton sk{};
  constexpr int NJ = 30;
  if (parents[0] != -1) return KIMODO_EINVAL;
  int depth[NJ] = {0}, max_depth = 0;
  for (int j = 0; j < NJ; ++j) {
    if (j > 0 && (parents[j] < 0 || parents[j] >= j)) return KIMODO_EINVAL;
    for (int k = 0; k < 3; ++k) {
      if (!std::isfinite(offsets[3 * j + k])) return KIMODO_EINVAL;
      sk.offset[j][k] = offsets[3 * j + k];
    }
    sk.parent[j] = parents[j];
    depth[j] = j ? depth[parents[j]] + 1 : 0;
    max_depth = std::max(max_depth, depth[j]);
  }
  while ((1 << sk.rounds) < max_depth + 1) ++sk.rounds;
  for (int j = 0; j < 32; ++j) sk.anc[0][j] = j > 0 && j < NJ ? parents[j] : -1;
  for (int r = 1; r < kmd::FK_MAX_ROUNDS; ++r)
    for (int j = 0; j < 32; ++j) sk.anc[r][j] = sk.anc[r - 1][j] >= 0 ? sk.anc[r - 1][sk.anc[r - 1][j]] : -1;
  if (n_frames == 0) return KIMODO_OK;
  if (kmd::fk_decode(motion, n_frames, sk, positions, rotations, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KIMODO_EHIP;
  return KIMODO_OK;
}

// Constraint sets (host only). A set covers key frames with one reference pose
// each; at a key frame it writes the features of its kind into the clip's
// known values and sets their mask bytes: the root path (x, z); the full body
// (the root stream and every joint's 9 features, contacts free); an end
// effector (the root stream and the 6D local rotations of the joints from the
// root joint to the end-effector joint, all that its forward kinematics reads).
kimodo_status kimodo_constraint_set(int32_t kind, int32_t T, int32_t n_keys, const int32_t *frames,
                                    const float *poses, int32_t joint, const int32_t *parents, float *known_values,
                                    uint8_t *known_mask) {
  constexpr int NJ = 30, JF = 9, ROT = 6;
  if (kind < KIMODO_CONSTRAINT_ROOT_PATH || kind > KIMODO_CONSTRAINT_END_EFFECTOR) return KIMODO_EINVAL;
  if (T < 1 || T > 4096 || n_keys < 0) return KIMODO_ESHAPE;
  if (n_keys == 0) return KIMODO_OK;
  if (!frames || !poses || !known_values || !known_mask) return KIMODO_EINVAL;
  for (int i = 0; i < n_keys; ++i)
    if (frames[i] < 0 || frames[i] >= T) return KIMODO_ESHAPE;
  bool cover[FEATS] = {};
  if (kind == KIMODO_CONSTRAINT_ROOT_PATH) {
    cover[0] = cover[2] = true;
  } else if (kind == KIMODO_CONSTRAINT_FULL_BODY) {
    for (int c = 0; c < ROOT + NJ * JF; ++c) cover[c] = true;
  } else {
    if (!parents || joint < 0 || joint >= NJ || parents[0] != -1) return KIMODO_EINVAL;
    for (int j = 1; j < NJ; ++j)
      if (parents[j] < 0 || parents[j] >= j) return KIMODO_EINVAL;
    for (int c = 0; c < ROOT; ++c) cover[c] = true;
    for (int j = joint; j >= 0; j = parents[j])
      for (int c = 0; c < ROT; ++c) cover[ROOT + JF * j + c] = true;
  }
  for (int i = 0; i < n_keys; ++i) {
    const size_t row = (size_t)frames[i] * FEATS;
    for (int c = 0; c < FEATS; ++c)
      if (cover[c]) {
        known_values[row + c] = poses[(size_t)i * FEATS + c];
        known_mask[row + c] = 1;
      }
  }
  return KIMODO_OK;
}

// The root path through n_points waypoints over n_frames frames: waypoint i
// at the real frame position i (n_frames - 1) / (n_points - 1), linear in
// between (in double, stored as float).
kimodo_status kimodo_root_path(int32_t n_points, const float *waypoints, int32_t n_frames, float *xz) {
  if (n_points < 1 || n_frames < 1 || n_frames > 4096) return KIMODO_ESHAPE;
  if (!waypoints || !xz) return KIMODO_EINVAL;
  for (int i = 0; i < 2 * n_points; ++i)
    if (!std::isfinite(waypoints[i])) return KIMODO_EINVAL;
  for (int f = 0; f < n_frames; ++f) {
    if (n_points == 1 || n_frames == 1) {
      xz[2 * f] = waypoints[0];
      xz[2 * f + 1] = waypoints[1];
      continue;
    }
    const double u = (double)f * (n_points - 1) / (n_frames - 1);
    const int seg = std::min((int)std::floor(u), n_points - 2);
    const double a = u - seg;
    for (int k = 0; k < 2; ++k) {
      const double w0 = waypoints[2 * seg + k], w1 = waypoints[2 * (seg + 1) + k];
      xz[2 * f + k] = (float)(w0 + a * (w1 - w0));
    }
  }
  return KIMODO_OK;
}

const char *kimodo_status_str(kimodo_status s) {
  switch (s) {
    case KIMODO_OK: return "ok";
    case KIMODO_EINVAL: return "invalid argument";
    case KIMODO_ESHAPE: return "shape out of range";
    case KIMODO_EDTYPE: return "unsupported dtype";
    case KIMODO_EWORKSPACE: return "workspace missing, misaligned or too small";
    case KIMODO_EWEIGHTS: return "weight table count or pointer invalid";
    case KIMODO_EHIP: return "HIP runtime error";
    case KIMODO_ESTATE: return "invalid context";
    case KIMODO_ECONFIG: return "unsupported model configuration";
  }
  return "unknown status";
}

const char *kimodo_last_error(const kimodo_ctx *ctx) { return ctx ? ctx->err.c_str() : ""; }

kimodo_status kimodo_graph_stats(const kimodo_ctx *ctx, int64_t *instantiated, int64_t *updated) {
  if (!ctx) return KIMODO_ESTATE;
  if (instantiated) *instantiated = ctx->graph_instantiations;
  if (updated) *updated = ctx->graph_updates;
  return KIMODO_OK;
}

void kimodo_destroy(kimodo_ctx *ctx) {
  if (!ctx) return;
  for (StepGraph &g : ctx->graphs) {
    if (g.done_recorded) (void)hipEventSynchronize(g.done);
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    if (g.graph) (void)hipGraphDestroy(g.graph);
    if (g.done) (void)hipEventDestroy(g.done);
  }
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  for (int j = 0; j < MAX_CHAINS - 1; ++j) {
    if (ctx->chain_stream[j]) (void)hipStreamDestroy(ctx->chain_stream[j]);
    if (ctx->join_event[j]) (void)hipEventDestroy(ctx->join_event[j]);
  }
  if (ctx->fork_event) (void)hipEventDestroy(ctx->fork_event);
  for (hipEvent_t e : ctx->events) (void)hipEventDestroy(e);
  delete ctx;
}

}  // extern "C"
