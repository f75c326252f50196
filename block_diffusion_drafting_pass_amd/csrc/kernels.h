// Internal interface between the C ABI (api.hip) and the gfx950 kernels
// (kernels.hip).  Not part of the public header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef uint16_t u16;

constexpr int kMaxSeqs = 128;
constexpr int kMaxHidden = 16384;  // widest hidden size the row kernels hold in registers
constexpr int kMaxKvLayers = 8;  // layers one all-layer K/V projection launch covers

// Per-call sequence table, passed to kernels by value.  Rows of sequence b in
// the current row space are [row_start[b], row_start[b+1]); row r of sequence
// b sits at position pos_base[b] + (r - row_start[b]) and its cache slot is
// slot_base[b] + position.
struct SeqTable {
  int32_t n;
  int32_t row_start[kMaxSeqs + 1];
  int32_t pos_base[kMaxSeqs];
  int32_t slot_base[kMaxSeqs];
};

// Weight-row maps: which weight row feeds column c (0..15) of 16-wide tile t.
enum MapKind : int {
  MAP_PLAIN = 0,   // row 16 t + c of w0
  MAP_SWIGLU = 1,  // c < 8: row 8 t + c of w0 (gate); c >= 8: row 8 t + c - 8 of w1 (up)
  MAP_QKV = 2,     // row 16 t + c of the stacked [w0; w1; w2] (q rows, k rows, v rows)
  MAP_KVL = 3,     // row 16 t + c of the stacked [wk_0; wv_0; wk_1; wv_1; ...] of all layers
};

// Epilogues applied to a finished 16x16 fp32 tile.
enum EpiKind : int {
  EPI_SWIGLU = 0,   // out_hi/lo[row][8 t + c] = hi/lo(silu(gate) * up)
  EPI_ARGMAX = 1,   // per-row (max, lowest index) key over the tile, optional logits
  EPI_PARTIAL = 2,  // out_f32[kc][row][16 t + c] = y (K chunk kc's share; rows < M)
  EPI_SAMPLE = 3,   // EPI_ARGMAX over logit / temp + Gumbel noise (sampled drafts; chosen
                    // by launch_gemm for EPI_ARGMAX launches with ep.temp > 0)
  EPI_RESID = 4,    // whole-K few-row GEMM only (rows < M): x[row][16 t + c] += y, then
                    // out_hi/lo[row][16 t + c] = hi/lo(gain * x) (not yet normalised) and
                    // ssq[row][t] = sum of x^2 over the tile's 16 columns
};

struct WeightSeg {
  const u16* w0;
  const u16* w1;
  const u16* w2;
  const u16* wk[kMaxKvLayers];  // MAP_KVL
  const u16* wv[kMaxKvLayers];
};

struct EpiParams {
  int M;          // valid rows
  int Mp;         // padded rows (plane stride of split outputs, row stride of partials)
  // EPI_PARTIAL
  float* out_f32;
  int ldo;
  // EPI_SWIGLU, EPI_RESID
  u16* out_hi;
  u16* out_lo;
  int ldh;
  // EPI_RESID: the residual rows x (row stride ldo, updated in place), the
  // next RMSNorm's gain, and the per-tile row sums of squares [Mp][n_tiles]
  float* x;
  const u16* gain;
  float* ssq;
  // EPI_SWIGLU after an EPI_RESID launch: the A rows are gain * x, not yet
  // normalised; each row's products are first scaled by RMSNorm's factor
  // 1 / sqrt(sum(ssq_in[row][0 .. n_ssq)) / norm_n + eps) (null: no scaling)
  const float* ssq_in;
  int n_ssq;
  int norm_n;
  float eps;
  // MAP_QKV / MAP_KVL
  int n_q, n_kv, head_dim;
  // EPI_ARGMAX: per-row argmax keys of each column tile (many-row GEMM) or of
  // each workgroup (few-row GEMM), [part][Mp]
  unsigned long long* amax_part;
  float* logits;                  // [n_seqs][block-1][vocab] or null
  int vocab;
  int block;
  // sampled drafts: temp > 0 replaces each logit l of draft row i of block b
  // by l / temp + G, G the Gumbel number of (seed, b, i, column)
  double temp;
  unsigned long long seed;
};

// Random-number purposes (the key's second word).
constexpr unsigned long long kPurposeDraft = 1, kPurposeAccept = 2, kPurposeResidual = 3;

struct GemmArgs {
  const u16* wpack;  // packed weights of this launch's mapped rows (few-row GEMM only), or null
  int pk_kmajor;     // wpack order: 0 tile-major (block (t, s) at t K/32 + s), 1 k-major (at s n_tiles + t)
  const u16* a_hi;   // A rows (bf16); with split A this is the hi plane
  const u16* a_lo;   // lo plane or null (single product)
  int lda;           // row stride of A in elements
  int a_rows;        // rows of A that exist in memory; others read as zero
  int K;
  int n_tiles;       // 16-wide output tiles in the mapped column space
  int q_rows;        // MAP_QKV: rows >= q_rows need no q columns (appended context rows); 0: all do
  WeightSeg w;
  int map;
  int epi;
  EpiParams ep;
};

// Launch shape of a GEMM over Mp padded rows: few rows (Mp <= 32) take the
// weight-streaming kernel with nc column tiles per wave and ks waves per
// workgroup; many rows (Mp a multiple of 128) the LDS-tiled one.  kc K
// chunks across workgroups (kc > 1 only with EPI_PARTIAL).  The same
// function sizes the partial buffers.
struct GemmPlan {
  int nc, kc, ks;
};
GemmPlan gemm_plan(int n_tiles, int K, int Mp, bool may_split);
constexpr int kSkinnyWaves = 4;  // waves per workgroup of the few-row GEMM
constexpr int kMaxKc = 16;       // most K chunks a GEMM is split into
// Padded row count of a GEMM operand: 16-row groups up to 32 rows (few-row
// kernel), else whole 128-row tiles.
inline int rows_pad(int m) { return m <= 32 ? (m + 15) / 16 * 16 : (m + 127) / 128 * 128; }

hipError_t launch_gemm(const GemmArgs& g, const SeqTable& st, int Mp, hipStream_t s);
// K chunks (1 or 2) of a many-row SwiGLU projection of n_tiles 16-column
// tiles; with 2, launch_gemm writes partial sums [2][Mp][16 n_tiles] fp32 to
// ep.out_f32 (which must then hold them) before the SwiGLU kernel.
int swiglu_kc(int n_tiles, int K, int Mp);
// Whether the whole-K few-row GEMM (EPI_RESID) takes this shape: 16 padded
// rows, K a multiple of 256 up to 4096, and at most 256 column tiles (the
// SwiGLU launch that follows reads a row's tile sums with one load per lane).
bool gemm_whole_k_fits(int n_tiles, int K, int Mp);

// Packed weights of one few-row GEMM launch: the launch's mapped weight rows
// (map, w, ep.n_q / n_kv / head_dim, n_tiles, K of g) rearranged so that
// column tile t, k-step s (32 k) is one contiguous 1 KB block in MFMA lane
// order: elements ((t K / 32 + s) 64 + lane) 8 .. + 7 hold mapped row
// 16 t + c, columns 32 s + 8 q .. + 7, for lane = 16 q + c.  A wave's weight
// loads then read 1 KB contiguous each.  Layout only: the GEMM over packed
// weights computes the same sums in the same order.
inline size_t packed_elems(int n_tiles, int K) { return (size_t)n_tiles * 16 * K; }
hipError_t launch_pack_weights(const GemmArgs& g, u16* dst, hipStream_t s);

// x[row] = E[token] (token: anchor for block row 0; for rows i >= 1 the mask
// id, or block_tokens[seq][i-1] when given), or
// x[row] += sum over kc of part[kc][row] (fixed kc order; part_rows = the
// partials' row stride per chunk); then out = hi/lo(gain * x / sqrt(mean(x^2)
// + eps)) for rows < M.  Rows M..out_rows-1 of out are zero, except in
// embedding mode with part given: there they are appended rows, out[row] =
// hi/lo(sum over kc of part[kc][row - M]) (no gain, no norm, x untouched).
hipError_t launch_resid_norm(float* x, const float* part, int kc, int part_rows, const int32_t* anchors,
                             const int32_t* block_tokens, const u16* embed, int block, int mask_id, int vocab,
                             const u16* gain, u16* out_hi, u16* out_lo, int H, int M, int out_rows, float eps,
                             hipStream_t s);
// out[row][j] = hi/lo(sum over kc of part[kc][row][j]) for rows < M (part_rows:
// the partials' row stride per chunk); rows M..out_rows-1 of out are zero.
hipError_t launch_reduce_split(const float* part, int kc, int part_rows, int N, u16* out_hi, u16* out_lo, int M,
                               int out_rows, hipStream_t s);
// Reduce q|k|v partials [kc][Mp][(n_q + 2 n_kv) d]; RoPE on q and k at each
// row's position; q -> q_hi/lo [row][n_q d] for rows < q_rows (later rows are
// appended context rows, which need only their K / V; the few-row GEMM leaves
// their q partials unwritten); k, v -> the layer's cache slots.
hipError_t launch_qkv_finish(const float* part, int kc, int M, int q_rows, int Mp, int n_q, int n_kv, int head_dim,
                             const float* rope_cos, const float* rope_sin, u16* q_hi, u16* q_lo,
                             u16* kv_cache, int64_t kv_tiles, const SeqTable& st, hipStream_t s);
// Reduce all-layer k|v partials [kc][Mp][n_layers 2 n_kv d]; RoPE on k;
// write every layer's cache slots.  layer_stride: elements between the
// caches of consecutive layers.
hipError_t launch_kv_finish(const float* part, int kc, int M, int Mp, int n_layers, int n_kv, int head_dim,
                            const float* rope_cos, const float* rope_sin, u16* kv_cache0, size_t layer_stride,
                            int64_t kv_tiles, const SeqTable& st, hipStream_t s);
// Blocks that share one context and one attention workgroup: member[g][j]
// is the j-th block of group g (-1 past the group's end).  Every member of a
// group has the same slot_base (the same context); the group's workgroup
// stages each context tile once for all of its members' query waves.
constexpr int kAttnGroup = 4;
struct AttnGroups {
  int32_t n;
  int16_t member[kMaxSeqs][kAttnGroup];
};
// Query heads one attention wave serves from each K / V fragment it reads
// (grouped launches), and the most blocks one group may hold at this shape
// (16 waves per workgroup, 8 when each wave serves two heads).
int attention_heads_per_wave(int n_q, int n_kv, bool grouped);
int attention_group_size(int n_q, int n_kv, int block);
// Block queries of sequence b (rows row_start[b] ..) against pos_base[b]
// context keys from its cache slots (slot_base[b] ..) and the block's own
// keys.  blk_kv null: the block keys follow the context keys in the cache;
// otherwise they are tile b of blk_kv (n_seqs tiles per kv head), and the
// cache is only read.  groups (only with blk_kv): one workgroup per group of
// blocks and kv head instead of per block and kv head.  max_tiles: key tiles
// of the longest unit (chooses the launch shape only).
hipError_t launch_attention(const u16* q_hi, const u16* q_lo, const u16* kv_cache, int64_t kv_tiles,
                            const u16* blk_kv, float* part_o, float* part_ml, u16* o_hi, u16* o_lo, int n_seqs,
                            int block, int n_q, int n_kv, int head_dim, int splits, int max_tiles,
                            const SeqTable& st, const AttnGroups* groups, hipStream_t s);
// Zero slots block .. kTileKeys-1 of the n_blocks x n_kv block tiles of a
// separate block K/V area (slots the block never writes; attention masks
// them, and zeros keep 0 * value finite).
hipError_t launch_clear_block_pad(u16* blk_kv, int n_blocks, int n_kv, int head_dim, int block, hipStream_t s);
// draft[b][i-1] from the largest key of block row i over n_parts partial keys.
hipError_t launch_argmax_reduce(const unsigned long long* part, int n_parts, int Mp, int n_seqs,
                                int block, int32_t* draft, hipStream_t s);
// Number of argmax partials the LM-head GEMM writes per row.
int argmax_parts(int n_tiles, int Mp);
hipError_t launch_accept(const int32_t* draft, const int32_t* target, int n, int block,
                         int32_t* accept, int32_t* next_anchor, hipStream_t s);
// Lossless verification of sampled blocks at temperature temp (fp64), with
// the vocabulary cut into verify_chunks(vocab) chunks: chunked log
// normalisers, then the keep tests, the first failing position and the
// residual / bonus sample, into accept / next_token.  scratch: 8-byte
// aligned, verify_scratch_bytes() bytes.
constexpr int kVerifyMaxChunks = 64;    // chunks of the log-normaliser pass (at most 4096 entries each)
constexpr int kVerifyMaxVocab = kVerifyMaxChunks * 4096;
constexpr int kVerifyMaxRChunks = 256;  // chunks of the residual / bonus sampling pass
size_t verify_scratch_bytes(int n, int block, int vocab);
hipError_t launch_verify_sample(const int32_t* draft, const float* q_logits, const float* p_logits, int n,
                                int block, int vocab, double temp, unsigned long long seed, void* scratch,
                                int32_t* accept, int32_t* next_token, hipStream_t s);

// Injected K/V cache layout of one layer.  Slots are grouped in tiles of
// kTileKeys; tile t of kv head g is one contiguous block of four planes:
//   K hi [kTileKeys][d], K lo [kTileKeys][d]      (key-major)
//   V hi [d][kTileKeys], V lo [d][kTileKeys]      (transposed)
// so a tile streams from HBM as 4 * kTileKeys * d bf16 values in one piece.
constexpr int kTileKeys = 64;
constexpr int kMaxSplits = 64;

__host__ __device__ inline size_t kv_tile_offset(int g, int64_t tile, int64_t kv_tiles, int d) {
  return ((size_t)g * kv_tiles + tile) * (size_t)(4 * kTileKeys * d);
}

// Key splits per (unit, kv head) for the attention pass: the call's tile work
// spread over the CUs, never more than there are tiles (unit_tiles: tiles
// summed over units and kv heads; grouped: units are groups of anchored
// blocks).  attention_max_splits bounds it for sizing the workspace.
int attention_splits(int pairs, int max_tiles, int64_t unit_tiles, bool grouped, int max_splits);
int attention_max_splits(int pairs);
size_t attention_partial_bytes(int n_seqs, int n_q, int qtiles, int splits, int head_dim);
size_t attention_ml_bytes(int n_seqs, int n_q, int qtiles, int splits);

}  // namespace dflash
