// C ABI of the DFlash draft pass: argument validation, context and workspace
// layout, and the launch sequence of each call.  Declared in include/dflash.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "dflash.h"
#include "kernels.h"

using namespace dflash;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(DFLASH_EHIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
// Rows of one fusion / K-V projection pass.  4096-row chunks give the
// many-row GEMMs whole 256-row tiles and long K loops without split-K
// (8192 positions: 3.12 ms with 1024-row chunks, 2.91 with 2048, 2.60 with
// 4096, 3.18 with 8192), at about 235 MB of workspace for the 5-layer
// hidden-4096 drafter.
constexpr int kIngestChunk = 4096;

size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }


struct LayerW {
  const u16 *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *wgate, *wup, *wdown;
};

int check_config(const dflash_config* c) {
  if (!c) return fail(DFLASH_EINVAL, "config is NULL");
  if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 ||
      c->intermediate < 1 || c->vocab < 1 || c->n_target_layers < 1)
    return fail(DFLASH_EINVAL, "config sizes must be positive");
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab)
    return fail(DFLASH_EINVAL, "mask_token_id %d outside [0, vocab)", c->mask_token_id);
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.0)) return fail(DFLASH_EINVAL, "rms_eps and rope_theta must be > 0");
  if (c->max_block < 2 || c->max_block > 32) return fail(DFLASH_EUNSUPPORTED, "max_block must be in [2, 32]");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(DFLASH_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (c->n_q_heads % c->n_kv_heads) return fail(DFLASH_ESHAPE, "n_q_heads must be a multiple of n_kv_heads");
  if (c->n_q_heads / c->n_kv_heads > 8) return fail(DFLASH_EUNSUPPORTED, "at most 8 query heads per kv head");
  if (c->hidden % 256 || c->intermediate % 256 || (c->n_q_heads * c->head_dim) % 256 ||
      ((int64_t)c->n_target_layers * c->hidden) % 256)
    return fail(DFLASH_EUNSUPPORTED, "hidden, intermediate, n_q_heads*head_dim and n_target_layers*hidden must be multiples of 256");
  if (c->vocab % 64) return fail(DFLASH_EUNSUPPORTED, "vocab must be a multiple of 64");
  if (c->hidden > kMaxHidden) return fail(DFLASH_EUNSUPPORTED, "hidden must be at most %d", kMaxHidden);
  return DFLASH_OK;
}

bool same_config(const dflash_config& a, const dflash_config& b) {
  return a.n_layers == b.n_layers && a.hidden == b.hidden && a.n_q_heads == b.n_q_heads &&
         a.n_kv_heads == b.n_kv_heads && a.head_dim == b.head_dim && a.intermediate == b.intermediate &&
         a.vocab == b.vocab && a.n_target_layers == b.n_target_layers && a.mask_token_id == b.mask_token_id &&
         a.max_block == b.max_block && a.rms_eps == b.rms_eps && a.rope_theta == b.rope_theta;
}

// Context layout: RoPE cos / sin tables, then per layer the tiled K/V cache
// (kv_tile_offset: per kv head, 64-slot tiles of K hi/lo and transposed V
// hi/lo planes).  Each sequence owns a whole number of tiles.
struct CtxLayout {
  std::vector<int64_t> slot_base;
  int64_t slots = 0;
  int64_t max_pos = 0;
  size_t cos_off = 0, sin_off = 0, kv_off = 0, layer_bytes = 0, total = 0;
};

int ctx_layout(const dflash_config* c, int32_t n_seqs, const int64_t* cap, CtxLayout* L) {
  if (n_seqs < 1 || n_seqs > kMaxSeqs) return fail(DFLASH_EUNSUPPORTED, "n_seqs must be in [1, %d]", kMaxSeqs);
  if (!cap) return fail(DFLASH_EINVAL, "capacity is NULL");
  L->slot_base.resize(n_seqs);
  int64_t slots = 0, max_pos = 0;
  for (int b = 0; b < n_seqs; ++b) {
    if (cap[b] < 0) return fail(DFLASH_EINVAL, "capacity[%d] < 0", b);
    const int64_t s = (cap[b] + c->max_block + kTileKeys - 1) / kTileKeys * kTileKeys;
    L->slot_base[b] = slots;
    slots += s;
    max_pos = std::max(max_pos, s);
  }
  if (slots >= (int64_t(1) << 30)) return fail(DFLASH_EUNSUPPORTED, "total context slots %lld too large", (long long)slots);
  L->slots = slots;
  L->max_pos = max_pos;
  const size_t half = c->head_dim / 2;
  L->cos_off = 0;
  L->sin_off = align_up(max_pos * half * sizeof(float));
  L->kv_off = L->sin_off + align_up(max_pos * half * sizeof(float));
  L->layer_bytes = align_up((size_t)4 * c->n_kv_heads * slots * c->head_dim * sizeof(u16));
  L->total = L->kv_off + (size_t)c->n_layers * L->layer_bytes;
  return DFLASH_OK;
}

struct WsLayout {
  int M = 0, Mp = 0, max_splits = 0, R = 0, Rp = 0;
  size_t x = 0, a_hi = 0, a_lo = 0, qa_hi = 0, qa_lo = 0, b_hi = 0, b_lo = 0, q_hi = 0, q_lo = 0, part_o = 0,
         part_ml = 0, amax = 0, part = 0, bkv = 0, draft_end = 0;
  size_t h_hi = 0, h_lo = 0, part_f = 0, ingest_end = 0;
  size_t total() const { return std::max(draft_end, ingest_end); }
};

// fp32 bytes of the K-chunk partial sums of one GEMM over Mp padded rows.
size_t part_bytes(int n_tiles, int K, int Mp, int N) {
  return (size_t)gemm_plan(n_tiles, K, Mp, true).kc * Mp * N * sizeof(float);
}

// Layers covered by one all-layer K/V projection launch.
int kv_group(const dflash_config* c) { return std::min(c->n_layers, kMaxKvLayers); }

WsLayout ws_layout(const dflash_config* c, int n_seqs, int block, int64_t max_new) {
  WsLayout W;
  const size_t H = c->hidden, I = c->intermediate, QD = (size_t)c->n_q_heads * c->head_dim;
  W.M = n_seqs * block;
  W.Mp = rows_pad(W.M);
  const int qtiles = (block + 15) / 16;
  // key splits of the attention pass: enough for one block per workgroup,
  // and for anchored blocks grouped attention_group_size to a workgroup
  // (fewer workgroups, so more splits)
  {
    const int gs = attention_group_size(c->n_q_heads, c->n_kv_heads, block);
    W.max_splits = std::max(attention_max_splits(n_seqs * c->n_kv_heads),
                            attention_max_splits((n_seqs + gs - 1) / gs * c->n_kv_heads));
  }
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align_up(bytes); return at; };
  const size_t Mp = W.Mp, wa = std::max(H, QD);
  // the q|k|v GEMM's rows: the block, plus appended positions on a fused step (<= 32 rows)
  const size_t Mq = Mp <= 32 ? 32 : Mp;
  W.x = take(Mp * H * 4);
  W.a_hi = take(Mp * wa * 2);
  W.a_lo = take(Mp * wa * 2);
  W.qa_hi = take(Mq * H * 2);
  W.qa_lo = take(Mq * H * 2);
  W.b_hi = take(Mp * I * 2);
  W.b_lo = take(Mp * I * 2);
  W.q_hi = take(Mq * QD * 2);
  W.q_lo = take(Mq * QD * 2);
  W.part_o = take(attention_partial_bytes(n_seqs, c->n_q_heads, qtiles, W.max_splits, c->head_dim));
  W.part_ml = take(attention_ml_bytes(n_seqs, c->n_q_heads, qtiles, W.max_splits));
  W.amax = take((size_t)(c->vocab / 16) * Mp * 8);
  {
    const int nqkv = (c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim, fw = c->n_target_layers * c->hidden;
    size_t pb = part_bytes(nqkv / 16, (int)H, (int)Mq, nqkv);
    pb = std::max(pb, part_bytes((int)H / 16, (int)QD, W.Mp, (int)H));
    pb = std::max(pb, part_bytes((int)H / 16, (int)I, W.Mp, (int)H));
    pb = std::max(pb, (size_t)swiglu_kc((int)I / 8, (int)H, W.Mp) * W.Mp * 2 * I * sizeof(float));
    if (W.Mp <= 32)
      for (int r = 16; r <= 32; r += 16)  // fusion of the appended rows on a fused step
        pb = std::max(pb, part_bytes((int)H / 16, fw, r, (int)H));
    W.part = take(pb);
  }
  // block K/V of anchored blocks: one cache-layout tile per block and kv head
  W.bkv = take((size_t)c->n_kv_heads * n_seqs * 4 * kTileKeys * c->head_dim * sizeof(u16));
  W.draft_end = o;
  o = 0;
  W.R = (int)std::min<int64_t>(std::max<int64_t>(max_new, 0), kIngestChunk);
  W.Rp = W.R > 0 ? rows_pad(W.R) : 0;
  W.h_hi = take((size_t)W.Rp * H * 2);
  W.h_lo = take((size_t)W.Rp * H * 2);
  if (W.R > 0) {
    // every chunk row count up to Rp (the last chunk may be shorter and split
    // K further), and every layer-group size (the last group may be smaller)
    const int fw = c->n_target_layers * c->hidden, kd2 = 2 * c->n_kv_heads * c->head_dim;
    size_t pb = 0;
    for (int r = 16; r <= W.Rp; r = r < 32 ? r + 16 : (r == 32 ? 128 : r + 128)) {
      pb = std::max(pb, part_bytes((int)H / 16, fw, r, (int)H));
      for (int nl = 1; nl <= kv_group(c); ++nl) pb = std::max(pb, part_bytes(nl * kd2 / 16, (int)H, r, nl * kd2));
    }
    W.part_f = take(pb);
  }
  W.ingest_end = o;
  return W;
}

}  // namespace

// Event pairs bracketing the launches of one stage (measurement only).
struct Probe {
  int stage = DFLASH_STAGE_NONE;
  std::vector<hipEvent_t> ev;  // start, stop, start, stop, ...
  int used = 0, missed = 0;

  void release() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    ev.clear();
    stage = DFLASH_STAGE_NONE;
    used = missed = 0;
  }
  bool on(int st) const { return stage == st; }
  void start(int st, hipStream_t s) {
    if (stage != st) return;
    if (2 * used < (int)ev.size()) (void)hipEventRecord(ev[2 * used], s);
  }
  void stop(int st, hipStream_t s) {
    if (stage != st) return;
    if (2 * used < (int)ev.size()) {
      (void)hipEventRecord(ev[2 * used + 1], s);
      ++used;
    } else {
      ++missed;
    }
  }
};

// Packed copies (dflash_model_pack) of the weights the few-row GEMM streams.
struct PackedLayer {
  const u16 *qkv = nullptr, *o = nullptr, *gate_up = nullptr, *down = nullptr;
};

struct dflash_model {
  dflash_config cfg;
  const u16* w_fc;
  const u16* embed;
  const u16* final_norm;
  std::vector<LayerW> layers;
  const u16* pk_fc = nullptr;  // packed fusion map, or null
  const u16* pk_lm = nullptr;  // packed LM head, or null
  std::vector<PackedLayer> pk_layers;
  mutable Probe probe;
  ~dflash_model() { probe.release(); }
};

struct dflash_ctx {
  dflash_config cfg;
  char* base;
  size_t bytes;
  int n_seqs;
  std::vector<int64_t> cap, len;
  CtxLayout L;
  u16* kv_cache(int l) const { return (u16*)(base + L.kv_off + (size_t)l * L.layer_bytes); }
  int64_t kv_tiles() const { return L.slots / kTileKeys; }
  const float* rope_cos() const { return (const float*)(base + L.cos_off); }
  const float* rope_sin() const { return (const float*)(base + L.sin_off); }
};

extern "C" {

const char* dflash_status_str(int s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_EINVAL: return "invalid argument";
    case DFLASH_ESHAPE: return "shape mismatch";
    case DFLASH_ECAPACITY: return "context capacity exceeded";
    case DFLASH_EWORKSPACE: return "workspace too small";
    case DFLASH_EALIGN: return "misaligned pointer";
    case DFLASH_EHIP: return "HIP runtime error";
    case DFLASH_EUNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

const char* dflash_last_error(void) { return g_last_error.c_str(); }

int32_t dflash_weight_count(const dflash_config* cfg) {
  if (!cfg || cfg->n_layers < 1) return -1;
  return 3 + 9 * cfg->n_layers;
}

int dflash_model_create(const dflash_config* cfg, const void* const* weights, dflash_model** out) {
  if (!out) return fail(DFLASH_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!weights) return fail(DFLASH_EINVAL, "weights is NULL");
  const int n = 3 + 9 * cfg->n_layers;
  for (int i = 0; i < n; ++i) {
    if (!weights[i]) return fail(DFLASH_EINVAL, "weights[%d] is NULL", i);
    if (!aligned(weights[i], 16)) return fail(DFLASH_EALIGN, "weights[%d] is not 16-byte aligned", i);
  }
  dflash_model* m = new (std::nothrow) dflash_model;
  if (!m) return fail(DFLASH_EINVAL, "out of host memory");
  m->cfg = *cfg;
  m->w_fc = (const u16*)weights[0];
  m->embed = (const u16*)weights[1];
  m->final_norm = (const u16*)weights[2];
  m->layers.resize(cfg->n_layers);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const void* const* w = weights + 3 + 9 * l;
    m->layers[l] = LayerW{(const u16*)w[0], (const u16*)w[1], (const u16*)w[2], (const u16*)w[3], (const u16*)w[4],
                          (const u16*)w[5], (const u16*)w[6], (const u16*)w[7], (const u16*)w[8]};
  }
  *out = m;
  return DFLASH_OK;
}

void dflash_model_destroy(dflash_model* m) { delete m; }

}  // extern "C"

namespace {

// The few-row GEMMs whose weights dflash_model_pack rearranges, in buffer
// order: the fusion map, the LM head, then per layer q|k|v, O, gate|up and
// down.  fn(args, which, layer) is called for each with the launch's weight
// map filled in.
enum PackSlot { PACK_FC, PACK_LM, PACK_QKV, PACK_O, PACK_GATE_UP, PACK_DOWN };

// Packed order per matrix.  The LM head, q|k|v and gate|up go k-major (the
// 1 KB blocks of one 32-k step of every column tile side by side), so that
// the workgroups at the same k stream one contiguous stretch together; the
// fusion map, O and down stay tile-major.  Measured over the few-row GEMM at
// 16 rows: LM head 220 -> 188 us (5.65 -> 6.62 TB/s), gate|up 37.6 -> 34.4,
// q|k|v 15.3 -> 14.3 us; O 8.4 -> 9.0 us, down and fusion unchanged.
constexpr int pack_kmajor(int which) { return which == PACK_LM || which == PACK_QKV || which == PACK_GATE_UP; }

template <typename F>
void for_each_packed(const dflash_model* m, F&& fn) {
  const dflash_config& c = m->cfg;
  const int H = c.hidden, QD = c.n_q_heads * c.head_dim, I = c.intermediate;
  auto args = [&](int map, int n_tiles, int K) {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.map = map;
    g.n_tiles = n_tiles;
    g.K = K;
    g.ep.n_q = c.n_q_heads;
    g.ep.n_kv = c.n_kv_heads;
    g.ep.head_dim = c.head_dim;
    return g;
  };
  GemmArgs g = args(MAP_PLAIN, H / 16, c.n_target_layers * H);
  g.w.w0 = m->w_fc;
  g.pk_kmajor = pack_kmajor(PACK_FC);
  fn(g, PACK_FC, -1);
  g = args(MAP_PLAIN, c.vocab / 16, H);
  g.w.w0 = m->embed;
  g.pk_kmajor = pack_kmajor(PACK_LM);
  fn(g, PACK_LM, -1);
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& Lw = m->layers[l];
    g = args(MAP_QKV, (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim / 16, H);
    g.w.w0 = Lw.wq;
    g.w.w1 = Lw.wk;
    g.w.w2 = Lw.wv;
    g.pk_kmajor = pack_kmajor(PACK_QKV);
    fn(g, PACK_QKV, l);
    g = args(MAP_PLAIN, H / 16, QD);
    g.w.w0 = Lw.wo;
    g.pk_kmajor = pack_kmajor(PACK_O);
    fn(g, PACK_O, l);
    g = args(MAP_SWIGLU, I / 8, H);
    g.w.w0 = Lw.wgate;
    g.w.w1 = Lw.wup;
    g.pk_kmajor = pack_kmajor(PACK_GATE_UP);
    fn(g, PACK_GATE_UP, l);
    g = args(MAP_PLAIN, H / 16, I);
    g.w.w0 = Lw.wdown;
    g.pk_kmajor = pack_kmajor(PACK_DOWN);
    fn(g, PACK_DOWN, l);
  }
}

size_t packed_bytes(const GemmArgs& g) { return align_up(packed_elems(g.n_tiles, g.K) * sizeof(u16)); }

}  // namespace

extern "C" {

size_t dflash_model_pack_bytes(const dflash_model* model) {
  if (!model) return 0;
  size_t total = 0;
  for_each_packed(model, [&](const GemmArgs& g, int, int) { total += packed_bytes(g); });
  return total;
}

int dflash_model_pack(dflash_model* model, void* dev_buf, size_t bytes, dflash_stream stream) {
  if (!model) return fail(DFLASH_EINVAL, "model is NULL");
  auto unpack = [&]() {
    model->pk_fc = model->pk_lm = nullptr;
    model->pk_layers.clear();
  };
  if (!dev_buf) {  // back to the row-major weights
    unpack();
    return DFLASH_OK;
  }
  if (!aligned(dev_buf, kAlign)) return fail(DFLASH_EALIGN, "dev_buf must be %zu-byte aligned", kAlign);
  const size_t need = dflash_model_pack_bytes(model);
  if (bytes < need) return fail(DFLASH_EWORKSPACE, "pack buffer holds %zu bytes, %zu needed", bytes, need);
  // the model switches to the packed copy only once every pack kernel has
  // been launched; on a launch error it keeps the row-major weights
  std::vector<PackedLayer> layers(model->layers.size());
  const u16 *fc = nullptr, *lm = nullptr;
  char* at = (char*)dev_buf;
  hipError_t e = hipSuccess;
  for_each_packed(model, [&](const GemmArgs& g, int which, int l) {
    if (e != hipSuccess) return;
    e = launch_pack_weights(g, (u16*)at, (hipStream_t)stream);
    const u16* p = (const u16*)at;
    switch (which) {
      case PACK_FC: fc = p; break;
      case PACK_LM: lm = p; break;
      case PACK_QKV: layers[l].qkv = p; break;
      case PACK_O: layers[l].o = p; break;
      case PACK_GATE_UP: layers[l].gate_up = p; break;
      default: layers[l].down = p; break;
    }
    at += packed_bytes(g);
  });
  if (e != hipSuccess) {
    unpack();
    return hip_fail(e, "model_pack: pack kernels");
  }
  model->pk_fc = fc;
  model->pk_lm = lm;
  model->pk_layers = std::move(layers);
  return DFLASH_OK;
}

size_t dflash_ctx_bytes(const dflash_config* cfg, int32_t n_seqs, const int64_t* capacity) {
  if (check_config(cfg)) return 0;
  CtxLayout L;
  if (ctx_layout(cfg, n_seqs, capacity, &L)) return 0;
  return L.total;
}

int dflash_ctx_create(const dflash_model* model, void* dev_buf, size_t bytes, int32_t n_seqs,
                      const int64_t* capacity, dflash_stream stream, dflash_ctx** out) {
  if (!out) return fail(DFLASH_EINVAL, "out is NULL");
  *out = nullptr;
  if (!model) return fail(DFLASH_EINVAL, "model is NULL");
  if (!dev_buf) return fail(DFLASH_EINVAL, "dev_buf is NULL");
  if (!aligned(dev_buf, kAlign)) return fail(DFLASH_EALIGN, "dev_buf is not 256-byte aligned");
  CtxLayout L;
  int rc = ctx_layout(&model->cfg, n_seqs, capacity, &L);
  if (rc) return rc;
  if (bytes < L.total) return fail(DFLASH_ECAPACITY, "context buffer holds %zu bytes, %zu needed", bytes, L.total);

  const dflash_config& c = model->cfg;
  const int half = c.head_dim / 2;
  std::vector<float> cs((size_t)L.max_pos * half), sn((size_t)L.max_pos * half);
  for (int64_t p = 0; p < L.max_pos; ++p)
    for (int j = 0; j < half; ++j) {
      const double ang = (double)p * pow(c.rope_theta, -2.0 * j / c.head_dim);
      cs[(size_t)p * half + j] = (float)cos(ang);
      sn[(size_t)p * half + j] = (float)sin(ang);
    }
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)dev_buf;
  hipError_t e = hipMemsetAsync(base + L.kv_off, 0, L.total - L.kv_off, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + L.cos_off, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + L.sin_off, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "dflash_ctx_create");

  dflash_ctx* x = new (std::nothrow) dflash_ctx;
  if (!x) return fail(DFLASH_EINVAL, "out of host memory");
  x->cfg = c;
  x->base = base;
  x->bytes = bytes;
  x->n_seqs = n_seqs;
  x->cap.assign(capacity, capacity + n_seqs);
  x->len.assign(n_seqs, 0);
  x->L = L;
  *out = x;
  return DFLASH_OK;
}

void dflash_ctx_destroy(dflash_ctx* ctx) { delete ctx; }

int64_t dflash_ctx_length(const dflash_ctx* ctx, int32_t seq) {
  if (!ctx || seq < 0 || seq >= ctx->n_seqs) return -1;
  return ctx->len[seq];
}

int dflash_ctx_truncate(dflash_ctx* ctx, int32_t seq, int64_t new_len) {
  if (!ctx) return fail(DFLASH_EINVAL, "ctx is NULL");
  if (seq < 0 || seq >= ctx->n_seqs) return fail(DFLASH_EINVAL, "seq %d outside [0, %d)", seq, ctx->n_seqs);
  if (new_len < 0 || new_len > ctx->len[seq])
    return fail(DFLASH_EINVAL, "new_len %lld outside [0, %lld]", (long long)new_len, (long long)ctx->len[seq]);
  ctx->len[seq] = new_len;
  return DFLASH_OK;
}

size_t dflash_workspace_bytes(const dflash_model* model, int32_t n_seqs, int32_t block, int64_t max_new_tokens) {
  if (!model || n_seqs < 1 || n_seqs > kMaxSeqs || block < 2 || block > model->cfg.max_block) return 0;
  return ws_layout(&model->cfg, n_seqs, block, max_new_tokens).total();
}

}  // extern "C"

namespace {

// Validate and enqueue an append (fusion, then every layer's injected K/V at
// positions length(b) ..) without changing any length: the caller advances
// the lengths once every launch of its call is enqueued.
int fuse_impl(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new, void* ws,
              size_t ws_bytes, hipStream_t s) {
  if (!model || !ctx) return fail(DFLASH_EINVAL, "model or ctx is NULL");
  if (!same_config(model->cfg, ctx->cfg)) return fail(DFLASH_ESHAPE, "ctx was created for another configuration");
  if (!n_new) return fail(DFLASH_EINVAL, "n_new is NULL");
  const dflash_config& c = model->cfg;
  int64_t total = 0;
  for (int b = 0; b < ctx->n_seqs; ++b) {
    if (n_new[b] < 0) return fail(DFLASH_EINVAL, "n_new[%d] < 0", b);
    if (ctx->len[b] + n_new[b] > ctx->cap[b])
      return fail(DFLASH_ECAPACITY, "sequence %d: length %lld + %d exceeds capacity %lld", b,
                  (long long)ctx->len[b], n_new[b], (long long)ctx->cap[b]);
    total += n_new[b];
  }
  if (total == 0) return DFLASH_OK;
  if (!features) return fail(DFLASH_EINVAL, "features is NULL");
  if (!aligned(features, 16)) return fail(DFLASH_EALIGN, "features is not 16-byte aligned");
  if (!ws) return fail(DFLASH_EINVAL, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(DFLASH_EALIGN, "workspace is not 256-byte aligned");
  const WsLayout W = ws_layout(&c, 1, 2, total);
  if (ws_bytes < W.ingest_end)
    return fail(DFLASH_EWORKSPACE, "workspace holds %zu bytes, %zu needed", ws_bytes, W.ingest_end);

  char* wsb = (char*)ws;
  u16* h_hi = (u16*)(wsb + W.h_hi);
  u16* h_lo = (u16*)(wsb + W.h_lo);
  float* part_f = (float*)(wsb + W.part_f);
  const int fw = c.n_target_layers * c.hidden;
  std::vector<int64_t> gstart(ctx->n_seqs + 1, 0);
  for (int b = 0; b < ctx->n_seqs; ++b) gstart[b + 1] = gstart[b] + n_new[b];

  for (int64_t r0 = 0; r0 < total; r0 += kIngestChunk) {
    const int R = (int)std::min<int64_t>(kIngestChunk, total - r0);
    const int Rp = rows_pad(R);
    SeqTable st;
    memset(&st, 0, sizeof(st));
    int n = 0;
    for (int b = 0; b < ctx->n_seqs; ++b) {
      const int64_t lo = std::max(gstart[b], r0), hi = std::min(gstart[b + 1], r0 + R);
      if (hi <= lo) continue;
      st.row_start[n] = (int32_t)(lo - r0);
      st.pos_base[n] = (int32_t)(ctx->len[b] + (lo - gstart[b]));
      st.slot_base[n] = (int32_t)ctx->L.slot_base[b];
      ++n;
    }
    st.n = n;
    st.row_start[n] = R;

    // fusion GEMM -> K-chunk partials -> h (hi/lo); then every layer's
    // W_k / W_v on h in one GEMM per layer group -> partials -> RoPE and the
    // cache write.
    GemmArgs f;
    memset(&f, 0, sizeof(f));
    f.a_hi = (const u16*)features + (size_t)r0 * fw;
    f.a_lo = nullptr;
    f.lda = fw;
    f.a_rows = R;
    f.K = fw;
    f.n_tiles = c.hidden / 16;
    f.w.w0 = model->w_fc;
    f.wpack = model->pk_fc;
    f.map = MAP_PLAIN;
    f.epi = EPI_PARTIAL;
    f.ep.M = R;
    f.ep.Mp = Rp;
    f.ep.out_f32 = part_f;
    f.ep.ldo = c.hidden;
    const int kcf = gemm_plan(f.n_tiles, f.K, Rp, true).kc;
    model->probe.start(DFLASH_STAGE_FUSION, s);
    hipError_t e = launch_gemm(f, st, Rp, s);
    if (e == hipSuccess) e = launch_reduce_split(part_f, kcf, Rp, c.hidden, h_hi, h_lo, R, Rp, s);
    model->probe.stop(DFLASH_STAGE_FUSION, s);
    if (e != hipSuccess) return hip_fail(e, "fuse_ctx: fusion GEMM");
    const int lg = kv_group(&c);
    for (int l0 = 0; l0 < c.n_layers; l0 += lg) {
      const int nl = std::min(lg, c.n_layers - l0);
      GemmArgs g;
      memset(&g, 0, sizeof(g));
      g.a_hi = h_hi;
      g.a_lo = h_lo;
      g.lda = c.hidden;
      g.a_rows = R;
      g.K = c.hidden;
      g.n_tiles = nl * 2 * c.n_kv_heads * c.head_dim / 16;
      for (int j = 0; j < nl; ++j) {
        g.w.wk[j] = model->layers[l0 + j].wk;
        g.w.wv[j] = model->layers[l0 + j].wv;
      }
      g.map = MAP_KVL;
      g.epi = EPI_PARTIAL;
      g.ep.M = R;
      g.ep.Mp = Rp;
      g.ep.n_kv = c.n_kv_heads;
      g.ep.head_dim = c.head_dim;
      g.ep.out_f32 = part_f;
      g.ep.ldo = g.n_tiles * 16;
      const int kck = gemm_plan(g.n_tiles, g.K, Rp, true).kc;
      model->probe.start(DFLASH_STAGE_KV_PROJ, s);
      e = launch_gemm(g, st, Rp, s);
      if (e == hipSuccess)
        e = launch_kv_finish(part_f, kck, R, Rp, nl, c.n_kv_heads, c.head_dim, ctx->rope_cos(), ctx->rope_sin(),
                             ctx->kv_cache(l0), ctx->L.layer_bytes / sizeof(u16), ctx->kv_tiles(), st, s);
      model->probe.stop(DFLASH_STAGE_KV_PROJ, s);
      if (e != hipSuccess) return hip_fail(e, "fuse_ctx: K/V projection");
    }
  }
  return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_fuse_ctx(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new,
                    void* ws, size_t ws_bytes, dflash_stream stream) {
  const int rc = fuse_impl(model, ctx, features, n_new, ws, ws_bytes, (hipStream_t)stream);
  if (rc) return rc;
  for (int b = 0; b < ctx->n_seqs; ++b) ctx->len[b] += n_new[b];
  return DFLASH_OK;
}

}  // extern "C"

namespace {

// Verified positions appended inside a draft pass (dflash_step): their fused
// features ride as extra rows of every layer's q|k|v GEMM, which reads the
// same W_k / W_v the separate context projection would.
struct Append {
  const u16* features = nullptr;  // [R][n_target_layers * hidden] bf16
  int R = 0;
  const int32_t* n_new = nullptr;  // host [n_seqs]
  const int64_t* old_len = nullptr;
};

// The blocks one draft pass drafts: block b sits at positions pos[b] ..
// pos[b] + block - 1 and sees the first pos[b] context keys of cache
// sequence seq[b].  sep: the blocks' own K/V go to the workspace and the
// cache is only read (several blocks may share a sequence); otherwise they
// go to the cache head-room right after the context (one block per
// sequence).
struct Blocks {
  int n = 0;
  int64_t pos[kMaxSeqs];
  int32_t seq[kMaxSeqs];
  bool sep = false;
};

// One block per sequence at positions lens[b] ..
Blocks seq_blocks(const dflash_ctx* ctx, const int64_t* lens) {
  Blocks bk;
  bk.n = ctx->n_seqs;
  for (int b = 0; b < bk.n; ++b) {
    bk.pos[b] = lens[b];
    bk.seq[b] = b;
  }
  return bk;
}

// tokens: NULL (mask tokens) or device [n][block-1] tokens for rows 1..block-1.
// smp: NULL (greedy drafts) or the sampling parameters of sampled drafts.
int draft_impl(const dflash_model* model, const dflash_ctx* ctx, const Blocks& bk, const int32_t* anchors,
               const int32_t* tokens, int block, int32_t* draft, float* logits, char* wsb, const WsLayout& W,
               hipStream_t s, const Append* ap, const dflash_sampling* smp = nullptr) {
  const dflash_config& c = model->cfg;
  const int n = bk.n;
  u16* bkv = (u16*)(wsb + W.bkv);
  float* x = (float*)(wsb + W.x);
  u16* a_hi = (u16*)(wsb + W.a_hi);
  u16* a_lo = (u16*)(wsb + W.a_lo);
  u16* qa_hi = (u16*)(wsb + W.qa_hi);
  u16* qa_lo = (u16*)(wsb + W.qa_lo);
  u16* b_hi = (u16*)(wsb + W.b_hi);
  u16* b_lo = (u16*)(wsb + W.b_lo);
  u16* q_hi = (u16*)(wsb + W.q_hi);
  u16* q_lo = (u16*)(wsb + W.q_lo);
  float* part_o = (float*)(wsb + W.part_o);
  float* part_ml = (float*)(wsb + W.part_ml);
  unsigned long long* amax = (unsigned long long*)(wsb + W.amax);
  float* part = (float*)(wsb + W.part);
  const int M = W.M, Mp = W.Mp, H = c.hidden, QD = c.n_q_heads * c.head_dim, I = c.intermediate;
  const int R = ap ? ap->R : 0;
  const int Mq = M + R, Mqp = rows_pad(Mq);  // rows of the q|k|v GEMM

  SeqTable st;  // block rows
  memset(&st, 0, sizeof(st));
  st.n = n;
  for (int b = 0; b < n; ++b) {
    st.row_start[b] = b * block;
    st.pos_base[b] = (int32_t)bk.pos[b];
    st.slot_base[b] = (int32_t)ctx->L.slot_base[bk.seq[b]];
  }
  st.row_start[n] = M;
  SeqTable sq = st;  // block rows, then the appended rows of each sequence at their own positions
  if (bk.sep)  // block b's row i -> slot b * kTileKeys + i of the workspace block area
    for (int b = 0; b < n; ++b) sq.slot_base[b] = b * kTileKeys - (int32_t)bk.pos[b];
  if (ap) {
    int e = n, off = M;
    for (int b = 0; b < n; ++b) {
      if (ap->n_new[b] == 0) continue;
      sq.row_start[e] = off;
      sq.pos_base[e] = (int32_t)ap->old_len[b];
      sq.slot_base[e] = (int32_t)ctx->L.slot_base[b];
      off += ap->n_new[b];
      ++e;
    }
    sq.n = e;
    sq.row_start[e] = off;
  }
  int max_tiles = 1, attn_units = n;
  int64_t unit_tiles = 0;
  AttnGroups groups;
  groups.n = 0;
  if (bk.sep) {
    // blocks of one sequence, in anchor order, share an attention workgroup
    // (up to attention_group_size of them): each context tile is read once
    // for the whole group
    const int gs = attention_group_size(c.n_q_heads, c.n_kv_heads, block);
    std::vector<int> order(n);
    for (int b = 0; b < n; ++b) order[b] = b;
    std::stable_sort(order.begin(), order.end(), [&](int u, int v) {
      return bk.seq[u] != bk.seq[v] ? bk.seq[u] < bk.seq[v] : bk.pos[u] < bk.pos[v];
    });
    int fill = gs;
    for (int i = 0; i < n; ++i) {
      const int b = order[i];
      if (fill == gs || bk.seq[groups.member[groups.n - 1][0]] != bk.seq[b]) {
        for (int j = 0; j < kAttnGroup; ++j) groups.member[groups.n][j] = -1;
        ++groups.n;
        fill = 0;
      }
      groups.member[groups.n - 1][fill++] = (int16_t)b;
    }
    for (int g = 0; g < groups.n; ++g) {
      int ct = 0, nb = 0;
      for (int j = 0; j < kAttnGroup && groups.member[g][j] >= 0; ++j, ++nb)
        ct = std::max<int>(ct, (int)((bk.pos[groups.member[g][j]] + kTileKeys - 1) / kTileKeys));
      max_tiles = std::max(max_tiles, ct + nb);
    }
    attn_units = groups.n;
  } else {
    for (int b = 0; b < n; ++b) {
      const int t = (int)((bk.pos[b] + block + kTileKeys - 1) / kTileKeys);
      max_tiles = std::max(max_tiles, t);
      unit_tiles += (int64_t)t * c.n_kv_heads;
    }
  }
  const int splits =
      attention_splits(attn_units * c.n_kv_heads, max_tiles, unit_tiles, bk.sep, W.max_splits);

  auto base_args = [&](const u16* ah, const u16* al, int lda, int K, int n_tiles, int epi, int map) {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.a_hi = ah;
    g.a_lo = al;
    g.lda = lda;
    g.a_rows = M;
    g.K = K;
    g.n_tiles = n_tiles;
    g.epi = epi;
    g.map = map;
    g.ep.M = M;
    g.ep.Mp = Mp;
    return g;
  };

  // The q|k|v, O and down GEMMs (and the fusion) may split K over
  // workgroups; the kernel that follows each sums the chunk partials in order
  // (RoPE + cache write, residual + RMSNorm, hi/lo split).
  const int nqkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int kc_qkv = gemm_plan(nqkv / 16, H, Mqp, true).kc;
  const int kc_o = gemm_plan(H / 16, QD, Mp, true).kc;
  // One 16-row block: the O projection runs whole-K and finishes the residual
  // and the MLP norm's gain in its epilogue; the gate|up GEMM applies the
  // norm's per-row factor.  That takes a reduce-and-normalise launch out of
  // every layer.  The projection's output rows go to the q|k|v input planes,
  // which are free between the q|k|v GEMM and the next layer's norm (rows
  // < M only: appended rows keep their fused features there).
  const bool whole_o = gemm_whole_k_fits(H / 16, QD, Mp);
  const int kc_d = gemm_plan(H / 16, I, Mp, true).kc;
  // the q|k|v GEMM reads its own A planes (block rows, then appended rows)
  u16* qin_hi = qa_hi;
  u16* qin_lo = qa_lo;
  hipError_t e;
  int fus_kc = 0, fus_rows = 0;

  if (ap) {
    // fused target features of the appended rows -> rows M .. M+R-1 of the q|k|v input
    const int fw = c.n_target_layers * H, Rp = rows_pad(R);
    GemmArgs f;
    memset(&f, 0, sizeof(f));
    f.a_hi = ap->features;
    f.lda = fw;
    f.a_rows = R;
    f.K = fw;
    f.n_tiles = H / 16;
    f.w.w0 = model->w_fc;
    f.wpack = model->pk_fc;
    f.map = MAP_PLAIN;
    f.epi = EPI_PARTIAL;
    f.ep.M = R;
    f.ep.Mp = Rp;
    f.ep.out_f32 = part;
    f.ep.ldo = H;
    fus_kc = gemm_plan(f.n_tiles, f.K, Rp, true).kc;
    fus_rows = Rp;
    model->probe.start(DFLASH_STAGE_FUSION, s);
    e = launch_gemm(f, st, Rp, s);
    model->probe.stop(DFLASH_STAGE_FUSION, s);
    if (e != hipSuccess) return hip_fail(e, "step: fusion GEMM");
  }

  if (bk.sep) {
    e = launch_clear_block_pad(bkv, n, c.n_kv_heads, c.head_dim, block, s);
    if (e != hipSuccess) return hip_fail(e, "draft: clear block K/V padding");
  }
  // block embedding + first norm for rows < M; with appended rows the same
  // launch sums their fusion partials into rows M .. M+R-1 of the q|k|v input
  e = launch_resid_norm(x, ap ? part : nullptr, fus_kc, fus_rows, anchors, tokens, model->embed, block,
                        c.mask_token_id, c.vocab, model->layers[0].attn_norm, qin_hi, qin_lo, H, M, M + R,
                        c.rms_eps, s);
  if (e != hipSuccess) return hip_fail(e, "draft_block: embed + attention norm");
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& Lw = model->layers[l];
    const PackedLayer Pw = model->pk_layers.empty() ? PackedLayer{} : model->pk_layers[l];
    GemmArgs g = base_args(qin_hi, qin_lo, H, H, nqkv / 16, EPI_PARTIAL, MAP_QKV);
    g.wpack = Pw.qkv;
    g.pk_kmajor = pack_kmajor(PACK_QKV);
    g.a_rows = Mq;
    g.q_rows = R > 0 ? M : 0;  // appended rows need only their K / V
    g.ep.M = Mq;
    g.ep.Mp = Mqp;
    g.ep.out_f32 = part;
    g.ep.ldo = nqkv;
    g.w.w0 = Lw.wq;
    g.w.w1 = Lw.wk;
    g.w.w2 = Lw.wv;
    g.ep.n_q = c.n_q_heads;
    g.ep.n_kv = c.n_kv_heads;
    g.ep.head_dim = c.head_dim;
    model->probe.start(DFLASH_STAGE_QKV, s);
    e = launch_gemm(g, st, Mqp, s);
    if (e == hipSuccess)
      e = launch_qkv_finish(part, kc_qkv, Mq, R > 0 ? M : Mq, Mqp, c.n_q_heads, c.n_kv_heads, c.head_dim, ctx->rope_cos(),
                            ctx->rope_sin(), q_hi, q_lo, bk.sep ? bkv : ctx->kv_cache(l),
                            bk.sep ? (int64_t)n : ctx->kv_tiles(), sq, s);
    model->probe.stop(DFLASH_STAGE_QKV, s);
    if (e != hipSuccess) return hip_fail(e, "draft_block: QKV projection");

    model->probe.start(DFLASH_STAGE_ATTENTION, s);
    e = launch_attention(q_hi, q_lo, ctx->kv_cache(l), ctx->kv_tiles(), bk.sep ? bkv : nullptr, part_o, part_ml,
                         a_hi, a_lo, n, block, c.n_q_heads, c.n_kv_heads, c.head_dim, splits, max_tiles, st, bk.sep ? &groups : nullptr, s);
    model->probe.stop(DFLASH_STAGE_ATTENTION, s);
    if (e != hipSuccess) return hip_fail(e, "draft_block: attention");

    g = base_args(a_hi, a_lo, QD, QD, H / 16, whole_o ? EPI_RESID : EPI_PARTIAL, MAP_PLAIN);
    g.w.w0 = Lw.wo;
    g.wpack = Pw.o;
    g.pk_kmajor = pack_kmajor(PACK_O);
    g.ep.ldo = H;
    if (whole_o) {
      g.ep.x = x;
      g.ep.gain = Lw.mlp_norm;
      g.ep.out_hi = qin_hi;
      g.ep.out_lo = qin_lo;
      g.ep.ldh = H;
      g.ep.ssq = part;
    } else {
      g.ep.out_f32 = part;
    }
    model->probe.start(DFLASH_STAGE_OPROJ, s);
    e = launch_gemm(g, st, Mp, s);
    model->probe.stop(DFLASH_STAGE_OPROJ, s);
    if (e != hipSuccess) return hip_fail(e, "draft_block: output projection");

    if (!whole_o) {
      e = launch_resid_norm(x, part, kc_o, Mp, nullptr, nullptr, nullptr, block, 0, c.vocab,
                            Lw.mlp_norm, a_hi, a_lo, H, M, M, c.rms_eps, s);
      if (e != hipSuccess) return hip_fail(e, "draft_block: MLP norm");
    }

    g = base_args(whole_o ? qin_hi : a_hi, whole_o ? qin_lo : a_lo, H, H, I / 8, EPI_SWIGLU, MAP_SWIGLU);
    g.w.w0 = Lw.wgate;
    g.w.w1 = Lw.wup;
    g.wpack = Pw.gate_up;
    g.pk_kmajor = pack_kmajor(PACK_GATE_UP);
    g.ep.out_hi = b_hi;
    g.ep.out_lo = b_lo;
    g.ep.ldh = I;
    g.ep.out_f32 = part;  // the K-chunk partials of a split many-row projection (swiglu_kc)
    if (whole_o) {
      g.ep.ssq_in = part;
      g.ep.n_ssq = H / 16;
      g.ep.norm_n = H;
      g.ep.eps = c.rms_eps;
    }
    model->probe.start(DFLASH_STAGE_GATE_UP, s);
    e = launch_gemm(g, st, Mp, s);
    model->probe.stop(DFLASH_STAGE_GATE_UP, s);
    if (e != hipSuccess) return hip_fail(e, "draft_block: gate/up projection");

    g = base_args(b_hi, b_lo, I, I, H / 16, EPI_PARTIAL, MAP_PLAIN);
    g.w.w0 = Lw.wdown;
    g.wpack = Pw.down;
    g.ep.out_f32 = part;
    g.ep.ldo = H;
    model->probe.start(DFLASH_STAGE_DOWN, s);
    e = launch_gemm(g, st, Mp, s);
    model->probe.stop(DFLASH_STAGE_DOWN, s);
    if (e != hipSuccess) return hip_fail(e, "draft_block: down projection");

    const bool last = l + 1 == c.n_layers;
    const u16* next_gain = last ? model->final_norm : model->layers[l + 1].attn_norm;
    e = launch_resid_norm(x, part, kc_d, Mp, nullptr, nullptr, nullptr, block, 0, c.vocab,
                          next_gain, last ? a_hi : qin_hi, last ? a_lo : qin_lo, H, M, M, c.rms_eps, s);
    if (e != hipSuccess) return hip_fail(e, "draft_block: residual + norm");
  }
  GemmArgs g = base_args(a_hi, a_lo, H, H, c.vocab / 16, EPI_ARGMAX, MAP_PLAIN);
  g.w.w0 = model->embed;
  g.wpack = model->pk_lm;
  g.pk_kmajor = pack_kmajor(PACK_LM);
  g.ep.amax_part = amax;
  g.ep.logits = logits;
  g.ep.vocab = c.vocab;
  g.ep.block = block;
  if (smp) {
    g.ep.temp = smp->temperature;
    g.ep.seed = smp->seed;
  }
  model->probe.start(DFLASH_STAGE_LM_HEAD, s);
  e = launch_gemm(g, st, Mp, s);
  model->probe.stop(DFLASH_STAGE_LM_HEAD, s);
  if (e != hipSuccess) return hip_fail(e, "draft_block: LM head");
  e = launch_argmax_reduce(amax, argmax_parts(c.vocab / 16, Mp), Mp, n, block, draft, s);
  if (e != hipSuccess) return hip_fail(e, "draft_block: argmax");
  return DFLASH_OK;
}

int check_draft_args(const dflash_model* model, const dflash_ctx* ctx, const int32_t* anchors, int32_t block,
                     int32_t* draft, float* logits, void* ws) {
  if (!model || !ctx) return fail(DFLASH_EINVAL, "model or ctx is NULL");
  if (!same_config(model->cfg, ctx->cfg)) return fail(DFLASH_ESHAPE, "ctx was created for another configuration");
  const dflash_config& c = model->cfg;
  if (block < 2 || block > c.max_block) return fail(DFLASH_EINVAL, "block %d outside [2, %d]", block, c.max_block);
  if (!anchors || !draft) return fail(DFLASH_EINVAL, "anchors or draft is NULL");
  if (!aligned(anchors, 4) || !aligned(draft, 4) || (logits && !aligned(logits, 4)))
    return fail(DFLASH_EALIGN, "anchors, draft and logits must be 4-byte aligned");
  if (!ws) return fail(DFLASH_EINVAL, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(DFLASH_EALIGN, "workspace is not 256-byte aligned");
  return DFLASH_OK;
}

int check_sampling(const dflash_sampling* sp) {
  if (!sp) return fail(DFLASH_EINVAL, "sampling parameters are NULL");
  if (!(sp->temperature > 0.0) || !std::isfinite(sp->temperature) || sp->temperature > 1e6)
    return fail(DFLASH_EINVAL, "temperature %g outside (0, 1e6]", sp->temperature);
  return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_draft_block(const dflash_model* model, const dflash_ctx* ctx, const int32_t* anchors, int32_t block,
                       int32_t* draft, float* logits, void* ws, size_t ws_bytes, dflash_stream stream) {
  int rc = check_draft_args(model, ctx, anchors, block, draft, logits, ws);
  if (rc) return rc;
  const WsLayout W = ws_layout(&model->cfg, ctx->n_seqs, block, 0);
  if (ws_bytes < W.draft_end)
    return fail(DFLASH_EWORKSPACE, "workspace holds %zu bytes, %zu needed", ws_bytes, W.draft_end);
  return draft_impl(model, ctx, seq_blocks(ctx, ctx->len.data()), anchors, nullptr, block, draft, logits, (char*)ws,
                    W, (hipStream_t)stream, nullptr);
}

int dflash_draft_sample(const dflash_model* model, const dflash_ctx* ctx, const int32_t* anchors, int32_t block,
                        const dflash_sampling* sampling, int32_t* draft, float* logits, void* ws, size_t ws_bytes,
                        dflash_stream stream) {
  int rc = check_draft_args(model, ctx, anchors, block, draft, logits, ws);
  if (rc) return rc;
  if ((rc = check_sampling(sampling))) return rc;
  const WsLayout W = ws_layout(&model->cfg, ctx->n_seqs, block, 0);
  if (ws_bytes < W.draft_end)
    return fail(DFLASH_EWORKSPACE, "workspace holds %zu bytes, %zu needed", ws_bytes, W.draft_end);
  return draft_impl(model, ctx, seq_blocks(ctx, ctx->len.data()), anchors, nullptr, block, draft, logits, (char*)ws,
                    W, (hipStream_t)stream, nullptr, sampling);
}

int dflash_draft_refine(const dflash_model* model, const dflash_ctx* ctx, const int32_t* anchors,
                        const int32_t* init_tokens, int32_t block, int32_t n_steps, int32_t* draft, float* logits,
                        void* ws, size_t ws_bytes, dflash_stream stream) {
  int rc = check_draft_args(model, ctx, anchors, block, draft, logits, ws);
  if (rc) return rc;
  if (n_steps < 1 || n_steps > 64) return fail(DFLASH_EINVAL, "n_steps %d outside [1, 64]", n_steps);
  if (init_tokens && !aligned(init_tokens, 4)) return fail(DFLASH_EALIGN, "init_tokens must be 4-byte aligned");
  const WsLayout W = ws_layout(&model->cfg, ctx->n_seqs, block, 0);
  if (ws_bytes < W.draft_end)
    return fail(DFLASH_EWORKSPACE, "workspace holds %zu bytes, %zu needed", ws_bytes, W.draft_end);
  // each pass reads its tokens in its first kernel and writes draft in its
  // last, so draft can carry the previous pass's drafts into the next pass
  const int32_t* toks = init_tokens;
  const Blocks bk = seq_blocks(ctx, ctx->len.data());
  for (int step = 0; step < n_steps; ++step) {
    rc = draft_impl(model, ctx, bk, anchors, toks, block, draft, step + 1 == n_steps ? logits : nullptr, (char*)ws, W,
                    (hipStream_t)stream, nullptr);
    if (rc) return rc;
    toks = draft;
  }
  return DFLASH_OK;
}

int dflash_draft_anchored(const dflash_model* model, const dflash_ctx* ctx, int32_t n_blocks,
                          const int32_t* block_seq, const int64_t* anchor_pos, const int32_t* anchors,
                          const int32_t* block_tokens, int32_t block, int32_t* draft, float* logits, void* ws,
                          size_t ws_bytes, dflash_stream stream) {
  int rc = check_draft_args(model, ctx, anchors, block, draft, logits, ws);
  if (rc) return rc;
  if (n_blocks < 1 || n_blocks > kMaxSeqs) return fail(DFLASH_EINVAL, "n_blocks %d outside [1, %d]", n_blocks, kMaxSeqs);
  if (!block_seq || !anchor_pos) return fail(DFLASH_EINVAL, "block_seq or anchor_pos is NULL");
  if (block_tokens && !aligned(block_tokens, 4)) return fail(DFLASH_EALIGN, "block_tokens must be 4-byte aligned");
  Blocks bk;
  bk.n = n_blocks;
  bk.sep = true;
  for (int j = 0; j < n_blocks; ++j) {
    const int32_t sq = block_seq[j];
    if (sq < 0 || sq >= ctx->n_seqs) return fail(DFLASH_EINVAL, "block_seq[%d] = %d outside [0, %d)", j, sq, ctx->n_seqs);
    if (anchor_pos[j] < 0 || anchor_pos[j] > ctx->len[sq])
      return fail(DFLASH_EINVAL, "anchor_pos[%d] = %lld outside [0, %lld] (length of sequence %d)", j,
                  (long long)anchor_pos[j], (long long)ctx->len[sq], sq);
    bk.pos[j] = anchor_pos[j];
    bk.seq[j] = sq;
  }
  const WsLayout W = ws_layout(&model->cfg, n_blocks, block, 0);
  if (ws_bytes < W.draft_end)
    return fail(DFLASH_EWORKSPACE, "workspace holds %zu bytes, %zu needed", ws_bytes, W.draft_end);
  return draft_impl(model, ctx, bk, anchors, block_tokens, block, draft, logits, (char*)ws, W, (hipStream_t)stream,
                    nullptr);
}

}  // extern "C"

namespace {

int step_impl(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new,
              const int32_t* anchors, int32_t block, const dflash_sampling* smp, int32_t* draft, float* logits,
              void* ws, size_t ws_bytes, dflash_stream stream) {
  int rc = check_draft_args(model, ctx, anchors, block, draft, logits, ws);
  if (rc) return rc;
  if (smp && (rc = check_sampling(smp))) return rc;
  if (!n_new) return fail(DFLASH_EINVAL, "n_new is NULL");
  const dflash_config& c = model->cfg;
  const int n = ctx->n_seqs;
  int64_t total = 0;
  for (int b = 0; b < n; ++b) {
    if (n_new[b] < 0) return fail(DFLASH_EINVAL, "n_new[%d] < 0", b);
    if (ctx->len[b] + n_new[b] > ctx->cap[b])
      return fail(DFLASH_ECAPACITY, "sequence %d: length %lld + %d exceeds capacity %lld", b,
                  (long long)ctx->len[b], n_new[b], (long long)ctx->cap[b]);
    total += n_new[b];
  }
  if (total > 0 && !features) return fail(DFLASH_EINVAL, "features is NULL");
  if (total > 0 && !aligned(features, 16)) return fail(DFLASH_EALIGN, "features is not 16-byte aligned");
  const WsLayout W = ws_layout(&c, n, block, total);
  if (ws_bytes < W.total()) return fail(DFLASH_EWORKSPACE, "workspace holds %zu bytes, %zu needed", ws_bytes, W.total());
  const int M = n * block;
  std::vector<int64_t> lens(n);
  for (int b = 0; b < n; ++b) lens[b] = ctx->len[b] + n_new[b];
  if (total == 0 || M > 32 || M + total > 32) {
    // too many rows for one fused weight sweep: append, then draft at the
    // new lengths; the lengths change only once both are enqueued
    rc = fuse_impl(model, ctx, features, n_new, ws, ws_bytes, (hipStream_t)stream);
    if (rc) return rc;
    rc = draft_impl(model, ctx, seq_blocks(ctx, lens.data()), anchors, nullptr, block, draft, logits, (char*)ws, W,
                    (hipStream_t)stream, nullptr, smp);
    if (rc) return rc;
    ctx->len = lens;
    return DFLASH_OK;
  }
  Append ap;
  ap.features = (const u16*)features;
  ap.R = (int)total;
  ap.n_new = n_new;
  ap.old_len = ctx->len.data();
  rc = draft_impl(model, ctx, seq_blocks(ctx, lens.data()), anchors, nullptr, block, draft, logits, (char*)ws, W,
                  (hipStream_t)stream, &ap, smp);
  if (rc) return rc;
  ctx->len = lens;
  return DFLASH_OK;
}

// Device scratch of dflash_step_noalloc.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code the array's name is
// only a stand-in for the symbol: device_scratch() asks the runtime for the
// current device's copy once per device (hipGetSymbolAddress) and every
// launch receives that pointer.
static __device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// This device's copy of `scratch` (the current device, which must be the
// stream's device).
int device_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "step_noalloc: hipGetDevice");
  if (s) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(s, &sd);
    if (e != hipSuccess) return hip_fail(e, "step_noalloc: hipStreamGetDevice");
    if (sd != dev) return fail(DFLASH_EINVAL, "stream belongs to device %d but device %d is current", (int)sd, dev);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(DFLASH_EUNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&d] { d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch)); });
  if (d.err != hipSuccess) return hip_fail(d.err, "step_noalloc: hipGetSymbolAddress");
  if (!d.ptr) return fail(DFLASH_EHIP, "step_noalloc: no address for the device scratch");
  *out = d.ptr;
  return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_step_noalloc(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new,
                        const int32_t* anchors, int32_t block, int32_t* draft, float* logits, dflash_stream stream) {
  // the size check comes first, so an oversized request never touches the device
  if (!model || !ctx) return fail(DFLASH_EINVAL, "model or ctx is NULL");
  if (!n_new) return fail(DFLASH_EINVAL, "n_new is NULL");
  if (block < 2 || block > model->cfg.max_block)
    return fail(DFLASH_EINVAL, "block %d outside [2, %d]", block, model->cfg.max_block);
  int64_t total = 0;
  for (int b = 0; b < ctx->n_seqs; ++b) {
    if (n_new[b] < 0) return fail(DFLASH_EINVAL, "n_new[%d] < 0", b);
    total += n_new[b];
  }
  const size_t need = ws_layout(&model->cfg, ctx->n_seqs, block, total).total();
  if (need > DFLASH_NOALLOC_SCRATCH_BYTES)
    return fail(DFLASH_EWORKSPACE, "this step needs %zu bytes of scratch; the static device scratch holds %zu", need,
                (size_t)DFLASH_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const int rc = device_scratch((hipStream_t)stream, &ws);
  if (rc) return rc;
  return step_impl(model, ctx, features, n_new, anchors, block, nullptr, draft, logits, ws,
                   DFLASH_NOALLOC_SCRATCH_BYTES, stream);
}

int dflash_step(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new,
                const int32_t* anchors, int32_t block, int32_t* draft, float* logits, void* ws, size_t ws_bytes,
                dflash_stream stream) {
  return step_impl(model, ctx, features, n_new, anchors, block, nullptr, draft, logits, ws, ws_bytes, stream);
}

int dflash_step_sample(const dflash_model* model, dflash_ctx* ctx, const void* features, const int32_t* n_new,
                       const int32_t* anchors, int32_t block, const dflash_sampling* sampling, int32_t* draft,
                       float* logits, void* ws, size_t ws_bytes, dflash_stream stream) {
  if (!sampling) return fail(DFLASH_EINVAL, "sampling parameters are NULL");
  return step_impl(model, ctx, features, n_new, anchors, block, sampling, draft, logits, ws, ws_bytes, stream);
}

size_t dflash_verify_workspace_bytes(int32_t n_seqs, int32_t block, int32_t vocab) {
  if (n_seqs < 0 || block < 2 || block > 1024 || vocab < 1 || vocab > kVerifyMaxVocab) return 0;
  return align_up(verify_scratch_bytes(n_seqs, block, vocab));
}

int dflash_verify_sample(const int32_t* draft, const float* draft_logits, const float* target_logits, int32_t n_seqs,
                         int32_t block, int32_t vocab, const dflash_sampling* sampling, int32_t* accept,
                         int32_t* next_token, void* ws, size_t ws_bytes, dflash_stream stream) {
  int rc = check_sampling(sampling);
  if (rc) return rc;
  if (n_seqs < 0) return fail(DFLASH_EINVAL, "n_seqs %d < 0", n_seqs);
  if (block < 2 || block > 1024) return fail(DFLASH_EINVAL, "block %d outside [2, 1024]", block);
  if (vocab < 1 || vocab > kVerifyMaxVocab)
    return fail(DFLASH_EINVAL, "vocab %d outside [1, %d]", vocab, kVerifyMaxVocab);
  if (n_seqs == 0) return DFLASH_OK;
  if (!draft || !draft_logits || !target_logits || !accept || !next_token || !ws)
    return fail(DFLASH_EINVAL, "a pointer argument is NULL");
  if (!aligned(draft, 4) || !aligned(draft_logits, 4) || !aligned(target_logits, 4) || !aligned(accept, 4) ||
      !aligned(next_token, 4))
    return fail(DFLASH_EALIGN, "arrays must be 4-byte aligned");
  if (!aligned(ws, 16)) return fail(DFLASH_EALIGN, "workspace must be 16-byte aligned");  // fp64 partials
  const size_t need = verify_scratch_bytes(n_seqs, block, vocab);
  if (ws_bytes < need) return fail(DFLASH_EWORKSPACE, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
  const hipError_t e = launch_verify_sample(draft, draft_logits, target_logits, n_seqs, block, vocab,
                                            sampling->temperature, sampling->seed, ws, accept, next_token,
                                            (hipStream_t)stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "verify_sample");
}

int dflash_probe_arm(dflash_model* model, int stage, int32_t max_launches) {
  if (!model) return fail(DFLASH_EINVAL, "model is NULL");
  if (stage <= DFLASH_STAGE_NONE || stage >= DFLASH_STAGE_COUNT) return fail(DFLASH_EINVAL, "stage %d unknown", stage);
  if (max_launches < 1 || max_launches > (1 << 20)) return fail(DFLASH_EINVAL, "max_launches %d outside [1, 2^20]", max_launches);
  Probe& p = model->probe;
  p.release();
  p.ev.reserve(2 * (size_t)max_launches);
  for (int i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t e;
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      p.release();
      return hip_fail(r, "probe_arm: hipEventCreate");
    }
    p.ev.push_back(e);
  }
  p.stage = stage;
  return DFLASH_OK;
}

int dflash_probe_read(dflash_model* model, double* total_ms, int32_t* launches, int32_t* missed) {
  if (!model || !total_ms || !launches) return fail(DFLASH_EINVAL, "model, total_ms or launches is NULL");
  Probe& p = model->probe;
  double sum = 0.0;
  for (int i = 0; i < p.used; ++i) {
    hipError_t r = hipEventSynchronize(p.ev[2 * i + 1]);
    float ms = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]);
    if (r != hipSuccess) {
      p.release();
      return hip_fail(r, "probe_read");
    }
    sum += ms;
  }
  *total_ms = sum;
  *launches = p.used;
  if (missed) *missed = p.missed;
  p.release();
  return DFLASH_OK;
}

int dflash_accept_len(const int32_t* draft, const int32_t* target, int32_t n_seqs, int32_t block, int32_t* accept,
                      int32_t* next_anchor, dflash_stream stream) {
  if (n_seqs < 0) return fail(DFLASH_EINVAL, "n_seqs < 0");
  if (block < 2 || block > 4096) return fail(DFLASH_EINVAL, "block %d outside [2, 4096]", block);
  if (n_seqs == 0) return DFLASH_OK;
  if (!draft || !target || !accept) return fail(DFLASH_EINVAL, "draft, target or accept is NULL");
  if (!aligned(draft, 4) || !aligned(target, 4) || !aligned(accept, 4) || (next_anchor && !aligned(next_anchor, 4)))
    return fail(DFLASH_EALIGN, "int32 arrays must be 4-byte aligned");
  hipError_t e = launch_accept(draft, target, n_seqs, block, accept, next_anchor, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "accept_len");
  return DFLASH_OK;
}

}  // extern "C"
