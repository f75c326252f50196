// gfx950 (MI355X, CDNA4) kernels of the DFlash block-diffusion draft pass.
//
// Precision scheme.  Weights are bf16 and enter the matrix cores unchanged.
// Every activation is an fp32 value carried as an unevaluated pair of bf16
// numbers hi + lo (hi = bf16(x), lo = bf16(x - hi)), so one fp32 x bf16
// product is two bf16 MFMAs into the same fp32 accumulator.  Attention needs
// fp32 x fp32 products (q.k and p.v), done as hi*hi + hi*lo + lo*hi.  The
// injected K/V cache stores its fp32 values as such pairs, in the layout the
// attention kernel feeds straight into MFMA registers.
//
// MFMA used throughout: v_mfma_f32_16x16x32_bf16.  A is 16 rows x 32 k, B is
// 32 k x 16 columns; lane l holds row / column (l % 16) and eight k values of
// group (l / 16); the 16x16 fp32 result gives lane l column (l % 16) and rows
// 4 (l / 16) + i, i = 0..3.  The k order inside a group never matters as long
// as A and B use the same one, which every kernel here does by construction.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace dflash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32; for every
// finite input it equals rounding the bit pattern at bit 16 with ties to
// even, denormals included).
__device__ __forceinline__ uint32_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two conversions in one instruction: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t bf16_rne2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi); x - hi is exact in fp32.
__device__ __forceinline__ void split_pair(float x, u16& hi, u16& lo) {
  const uint32_t h = bf16_rne(x);
  hi = (u16)h;
  lo = (u16)bf16_rne(x - bf16_val(h));
}

// 2^x on the hardware exponential unit (softmax weights: x <= 0; -inf -> 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 ld_frag(const u16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
// Streaming load of a weight fragment that is read once (non-temporal hint).
__device__ __forceinline__ bf16x8 ld_frag_stream(const u16* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
// 16-byte load with the non-temporal hint: cache tiles that a workgroup with
// splits of many tiles streams once (32 sequences of 2048 keys: draft pass
// 3.651 -> 3.571 ms; 8192 keys 0.725 -> 0.719 ms, same box).  Splits of one
// tile keep plain loads (context 1024: 0.664 -> 0.668 ms with the hint).
__device__ __forceinline__ u32x4 ld_tile_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ bf16x8 zero_frag() {
  const u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight fp32 values -> two bf16x8 fragments (hi and lo parts).
__device__ __forceinline__ void split_frag(const float* v, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = bf16_rne2(v[2 * j], v[2 * j + 1]);
    l[j] = bf16_rne2(v[2 * j] - bf16_val(h[j] & 0xFFFFu), v[2 * j + 1] - bf16_val(h[j] >> 16));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// Max / sum of v over lanes l and l ^ 16 (l ^ 32).  The gfx950 lane-swap
// instructions hand every lane both values in registers, without the LDS
// round trip of a shuffle; the pair comes in either order, and max and + are
// commutative, so the results equal those of an xor shuffle by m bit for bit.
template <int M>
__device__ __forceinline__ void xor_pair(float v, float& a, float& b) {
  static_assert(M == 16 || M == 32, "lane swaps exist for 16 and 32");
  const uint32_t u = __float_as_uint(v);
  const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
template <int M>
__device__ __forceinline__ float max_xor(float v) {
  float a, b;
  xor_pair<M>(v, a, b);
  return fmaxf(a, b);
}
template <int M>
__device__ __forceinline__ float sum_xor(float v) {
  float a, b;
  xor_pair<M>(v, a, b);
  return a + b;
}

// Largest 64-bit key over the 16 lanes of each row of a wave, every lane of
// the row ending with it, by DPP lane permutations (no LDS round trips):
// quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), the mirror
// within 8 lanes, the mirror within 16.  Max is order-independent, so any
// pairing that reaches every lane gives the same key.
template <int CTRL>
__device__ __forceinline__ u64 dpp_u64(u64 v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ u64 max_u64(u64 a, u64 b) { return a > b ? a : b; }
__device__ __forceinline__ u64 max_row16_u64(u64 k) {
  k = max_u64(k, dpp_u64<0xB1>(k));
  k = max_u64(k, dpp_u64<0x4E>(k));
  k = max_u64(k, dpp_u64<0x141>(k));
  return max_u64(k, dpp_u64<0x140>(k));
}
// ... over the whole wave: the rows' keys then meet by the lane swaps (both
// halves of a key move by the same lane mapping)
__device__ __forceinline__ u64 max_wave_u64(u64 k) {
  k = max_row16_u64(k);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
    const auto rl = half == 0 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                              : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto rh = half == 0 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                              : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    k = max_u64(((u64)rh[0] << 32) | rl[0], ((u64)rh[1] << 32) | rl[1]);
  }
  return k;
}

// Sum / max of v over the 64 lanes of a wave, every lane ending with the same
// bits: the DPP butterflies above within each 16-lane row, then the lane
// swaps across rows.  The pairing is fixed and + and max are commutative, so
// the result depends only on the 64 inputs.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum_row16(float v) {  // ... over each 16-lane row only
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  return v + dpp_f32<0x140>(v);
}
__device__ __forceinline__ float sum_wave(float v) { return sum_xor<32>(sum_xor<16>(sum_row16(v))); }
__device__ __forceinline__ float max_wave(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return max_xor<32>(max_xor<16>(v));
}

// Sequence owning `row` in the current row space (row_start is ascending).
__device__ __forceinline__ int seq_of_row(const SeqTable& st, int row) {
  int b = 0;
  for (int j = 1; j < st.n; ++j)
    if (row >= st.row_start[j]) b = j;
  return b;
}

// Order-preserving key of an fp32 value (finite inputs), packed with the
// complemented column so that a u64 max picks the largest value and, among
// equal values, the lowest column.
__device__ __forceinline__ u64 argmax_key(float v, int col) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((u64)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)col);
}

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds, each
// multiplying words 0 and 2 by the round constants and mixing the 128-bit
// products' halves with words 1 and 3 and the key, which is then advanced by
// the Weyl constants.  Returns the four output words.
__device__ __forceinline__ void philox4(u64 c0, u64 c1, u64 c2, u64 c3, u64 k0, u64 k1, u64 (&out)[4]) {
  constexpr u64 M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr u64 W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const u64 hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const u64 hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

__device__ __forceinline__ double word_uniform(u64 w) { return ((double)(w >> 11) + 0.5) * 0x1.0p-53; }

// Uniform number in (0, 1) of (seed, purpose, block b, position i, index v):
// the top 53 bits of word i mod 4 of the Philox block at counter
// (v, i div 4, b, 0), key (seed, purpose).
__device__ __forceinline__ double philox_uniform(u64 seed, u64 purpose, int b, int i, int v) {
  u64 w[4];
  philox4((u64)v, (u64)(i >> 2), (u64)b, 0ull, seed, purpose, w);
  return word_uniform(w[i & 3]);
}

__device__ __forceinline__ double gumbel(double u) { return -log(-log(u)); }

// The same Gumbel number of word w in float32: -log(U) is formed from U for
// U < 1/2 and as -log1p(-(1 - U)) above, with 1 - U exact from the integer,
// so it keeps full relative precision where U is close to 1.
__device__ __forceinline__ float gumbel_f32(u64 w) {
  const u64 m = w >> 11;                                    // U = (m + 1/2) 2^-53
  const double one_minus = ((double)((1ull << 53) - m) - 0.5) * 0x1.0p-53;
  const float e = m < (1ull << 52) ? -logf((float)(((double)m + 0.5) * 0x1.0p-53))
                                   : -log1pf(-(float)one_minus);
  return -logf(e);
}

// The values whose per-row argmax are the drafts, for a lane's four rows
// row0 .. row0 + 3 at one column: the logits themselves (greedy), or
// logit / temp + Gumbel noise (a sample from softmax(logits / temp)), in
// float32 like the logits; one Philox block serves the rows that share a
// (block, position div 4).
template <bool SAMPLE>
__device__ __forceinline__ f32x4 draft_scores(const EpiParams& ep, int row0, int col, f32x4 v) {
  if constexpr (!SAMPLE) return v;
  const float inv_t = (float)(1.0 / ep.temp);
  u64 w[4];
  int cur = -1;
  f32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + i, b = row / ep.block, pos = row % ep.block;
    const int key = b * 1024 + (pos >> 2);
    if (key != cur) {
      philox4((u64)col, (u64)(pos >> 2), (u64)b, 0ull, ep.seed, kPurposeDraft, w);
      cur = key;
    }
    out[i] = v[i] * inv_t + gumbel_f32(w[pos & 3]);
  }
  return out;
}

// ---------------------------------------------------------------------------
// weight-row maps and epilogues (shared by both GEMM kernels)
// ---------------------------------------------------------------------------

template <int MAP>
__device__ __forceinline__ const u16* weight_row(const WeightSeg& w, const EpiParams& ep, int tile,
                                                 int c, int K) {
  if (MAP == MAP_PLAIN) return w.w0 + (size_t)(tile * 16 + c) * K;
  if (MAP == MAP_SWIGLU) return (c < 8 ? w.w0 : w.w1) + (size_t)(tile * 8 + (c & 7)) * K;
  if (MAP == MAP_QKV) {
    const int r = tile * 16 + c, qd = ep.n_q * ep.head_dim, kd = ep.n_kv * ep.head_dim;
    if (r < qd) return w.w0 + (size_t)r * K;
    if (r < qd + kd) return w.w1 + (size_t)(r - qd) * K;
    return w.w2 + (size_t)(r - qd - kd) * K;
  }
  // MAP_KVL
  const int kd = ep.n_kv * ep.head_dim, r = tile * 16 + c;
  const int l = r / (2 * kd), rr = r % (2 * kd);
  return rr < kd ? w.wk[l] + (size_t)rr * K : w.wv[l] + (size_t)(rr - kd) * K;
}

// Position of a row and its injected-cache element address helpers.
__device__ __forceinline__ u16* kv_k_elem(u16* cache, int gk, int64_t slot, int64_t kv_tiles, int d, int col) {
  return cache + kv_tile_offset(gk, slot / kTileKeys, kv_tiles, d) + (slot % kTileKeys) * d + col;
}
__device__ __forceinline__ u16* kv_v_elem(u16* cache, int gk, int64_t slot, int64_t kv_tiles, int d, int col) {
  return cache + kv_tile_offset(gk, slot / kTileKeys, kv_tiles, d) + 2 * kTileKeys * d + col * kTileKeys +
         slot % kTileKeys;
}

// LM-head tile: for this lane's rows r0 + 4 (lane / 16) + i, the largest
// draft score over the tile's 16 columns (lowest column on ties) as an
// order-preserving key, 0 for rows that draft nothing; logits are written on
// the way when asked for.  All 64 lanes must call this together.
template <bool SAMPLE>
__device__ __forceinline__ void argmax_tile_keys(const EpiParams& ep, int tile, int r0, f32x4 v, int lane,
                                                 u64 (&key)[4]) {
  const int c = lane & 15, g = lane >> 4;
  const int col = tile * 16 + c;
  const f32x4 sc = draft_scores<SAMPLE>(ep, r0 + 4 * g, col, v);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + 4 * g + i;
    const int bi = row % ep.block;
    const bool draft_row = row < ep.M && bi != 0;
    if (draft_row && ep.logits)
      ep.logits[((size_t)(row / ep.block) * (ep.block - 1) + (bi - 1)) * ep.vocab + col] = v[i];
    key[i] = max_row16_u64(draft_row ? argmax_key(sc[i], col) : 0ull);
  }
}

// v: the 16x16 fp32 tile in MFMA result layout (lane: column c = lane % 16,
// rows r0 + 4 (lane / 16) + i).  All 64 lanes must call this together.
// kc: the K chunk this tile sums (EPI_PARTIAL only).
template <int EPI>
__device__ __forceinline__ void epilogue(const EpiParams& ep, const SeqTable& st, int tile, int r0,
                                         f32x4 v, int lane, int kc) {
  (void)st;
  const int c = lane & 15, g = lane >> 4;
  if (EPI == EPI_PARTIAL) {
    const int col = tile * 16 + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 4 * g + i;
      if (row < ep.M) ep.out_f32[((size_t)kc * ep.Mp + row) * ep.ldo + col] = v[i];
    }
  } else if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float up = dpp_f32<0x128>(v[i]);  // lane c+8 holds the up projection (DPP row_ror:8: lane ^ 8)
      const int row = r0 + 4 * g + i;
      if (c < 8 && row < ep.Mp) {
        u16 h = 0, l = 0;
        if (row < ep.M) {
          const float gt = v[i];
          split_pair(gt / (1.0f + expf(-gt)) * up, h, l);
        }
        const size_t o = (size_t)row * ep.ldh + tile * 8 + c;
        ep.out_hi[o] = h;
        ep.out_lo[o] = l;
      }
    }
  } else if (EPI == EPI_ARGMAX || EPI == EPI_SAMPLE) {
    u64 key[4];
    argmax_tile_keys<EPI == EPI_SAMPLE>(ep, tile, r0, v, lane, key);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 4 * g + i;
      if (c == 0 && row < ep.Mp) ep.amax_part[(size_t)tile * ep.Mp + row] = key[i];
    }
  }
}

// LM-head tail of the few-row GEMM.  Per draft row, the largest logit of the
// workgroup's tiles (lowest column on ties) as an order-preserving 64-bit key,
// combined in LDS (max is order-independent, so the result is deterministic)
// and stored as this workgroup's partial; a small kernel reduces the
// partials.  Logits are written on the way when asked for.
template <int RG, int NC, int KS, bool SAMPLE>
__device__ __forceinline__ void argmax_tail(const EpiParams& ep, int tile0, f32x4 (*red)[RG * NC][64], int lane,
                                            int ks) {
  __shared__ u64 rk[RG * 16];
  const int c = lane & 15, g = lane >> 4;
  if (threadIdx.x < RG * 16) rk[threadIdx.x] = 0;
  __syncthreads();
  for (int it = ks; it < RG * NC; it += KS) {
    f32x4 s = red[0][it][lane];
#pragma unroll
    for (int q = 1; q < KS; ++q) s += red[q][it][lane];
    const int col = (tile0 + it % NC) * 16 + c, r0 = (it / NC) * 16;
    const f32x4 sc = draft_scores<SAMPLE>(ep, r0 + 4 * g, col, s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 4 * g + i;
      const int bi = row % ep.block;
      const bool draft_row = row < ep.M && bi != 0;
      if (draft_row && ep.logits)
        ep.logits[((size_t)(row / ep.block) * (ep.block - 1) + (bi - 1)) * ep.vocab + col] = s[i];
      const u64 key = max_row16_u64(draft_row ? argmax_key(sc[i], col) : 0ull);
      if (c == 0 && key) atomicMax(&rk[row], key);
    }
  }
  __syncthreads();
  if (threadIdx.x < RG * 16 && (int)threadIdx.x < ep.Mp)
    ep.amax_part[(size_t)blockIdx.x * ep.Mp + threadIdx.x] = rk[threadIdx.x];
}

// ---------------------------------------------------------------------------
// Skinny weight-streaming GEMM: Y[M<=32][N] = A[M][K] W^T, W [N][K] bf16.
// Workgroup (x, y) owns NC 16-column tiles and K chunk y of gridDim.y; its
// KS waves (four; eight for narrow split-K outputs and the SwiGLU
// projection) split the chunk.  PK:
// the weights come packed (launch_pack_weights), so every weight load reads
// 1 KB contiguous per wave, with the non-temporal hint (read once); in the
// k-major order the NC tiles of one k-step are adjacent too, and workgroups
// at the same k read one stretch together.  Each wave streams its NC weight-row
// slices straight into MFMA B registers (16 B per lane per tile and k-step,
// two 32-k steps per batch, the next batch in flight while the current one
// is multiplied) and reuses every A fragment for all NC tiles.  Partial sums
// meet in LDS in a fixed order; the tiles' epilogues are spread over the
// waves.  With several K chunks the epilogue is EPI_PARTIAL and a later
// kernel sums the chunks in order.
// ---------------------------------------------------------------------------

template <int EPI, int MAP, int NC, int RG, bool SPLIT, int KS, bool PK>
__device__ __forceinline__ void skinny_body(const GemmArgs& ga, const SeqTable& st, int tile0, int kc, int nkc) {
  constexpr int U = 2;
  // packed weights: one 1 KB block per (tile, 32 k); k advances 16 elements
  // per k tile-major, 16 n_tiles k-major
  const size_t KM = PK ? (ga.pk_kmajor ? (size_t)16 * ga.n_tiles : 16) : 1;
  const size_t TM = ga.pk_kmajor ? 1 : ga.K / 32;  // blocks per tile step
  const int lane = threadIdx.x & 63, ks = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int kw = ga.K / (nkc * KS);
  const int kb = (kc * KS + ks) * kw, ke = kb + kw;

  const u16* wp[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j)
    wp[j] = PK ? ga.wpack + ((size_t)(tile0 + j) * TM * 64 + lane) * 8
               : weight_row<MAP>(ga.w, ga.ep, tile0 + j, c, ga.K) + g * 8;
  auto ldw = [&](int j, int k) { return PK ? ld_frag_stream(wp[j] + (size_t)k * KM) : ld_frag(wp[j] + k); };
  // Rows past a_rows read row a_rows - 1 instead: an output row depends only
  // on its own A row, and no epilogue consumes rows >= M (M <= a_rows).
  const u16* ah[RG];
  const u16* al[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int row = min(rg * 16 + c, ga.a_rows - 1);
    ah[rg] = ga.a_hi + (size_t)row * ga.lda + g * 8;
    al[rg] = SPLIT ? ga.a_lo + (size_t)row * ga.lda + g * 8 : nullptr;
  }
  // SwiGLU over gain * x rows not yet normalised (ep.ssq_in; one row group):
  // wave ks's rows ks, ks + KS, .. load their per-tile sums of squares ahead
  // of the weights and reduce them once the products are done
  constexpr bool NORM = EPI == EPI_SWIGLU && RG == 1;
  constexpr int NRW = NORM ? (16 + KS - 1) / KS : 1;
  const bool norm = NORM && ga.ep.ssq_in != nullptr;
  f32x4 sqv[NRW];
#pragma unroll
  for (int j = 0; j < NRW; ++j) {
    sqv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int row = ks + KS * j;
    if (norm && row < RG * 16 && lane * 4 < ga.ep.n_ssq)
      sqv[j] = *reinterpret_cast<const f32x4*>(ga.ep.ssq_in + (size_t)row * ga.ep.n_ssq + lane * 4);
  }
  f32x4 acc[RG][NC];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[rg][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // row groups that need none of this workgroup's columns (appended context
  // rows against q columns) skip their products; their partials stay zero
  int rg_end = RG;
  if (MAP == MAP_QKV && RG > 1 && ga.q_rows > 0 && (tile0 + NC) * 16 <= ga.ep.n_q * ga.ep.head_dim)
    rg_end = (ga.q_rows + 15) / 16;

  // A fragments travel one batch ahead with the weights: loads complete in
  // issue order, so a batch's A loaded after the next batch's weights would
  // make every wave wait for those weights before multiplying (16 rows: LM
  // head 187 -> 183 us, gate|up 35.7 -> 33.5 us; 32 rows: LM head 263 -> 222,
  // gate|up 39.1 -> 37.2 us).  Two row groups of split-K partial outputs (the
  // q|k|v, O and down projections) and eight-tile, eight-wave shapes load A
  // in the multiply: there the extra registers cost occupancy or spill.
  constexpr bool APF = RG == 1 || (EPI != EPI_PARTIAL && !(NC == 8 && KS == 8));
  constexpr int NPL = SPLIT ? 2 : 1;
  auto lda_ = [&](int pl, int rg, int k) { return ld_frag((pl ? al[rg] : ah[rg]) + k); };
  bf16x8 wf[U][NC], af[APF ? U : 1][RG][NPL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (APF)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl)
          if (rg < rg_end) af[u][rg][pl] = lda_(pl, rg, kb + u * 32);
#pragma unroll
    for (int j = 0; j < NC; ++j) wf[u][j] = ldw(j, kb + u * 32);
  }
  auto multiply = [&](int k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        if (rg >= rg_end) break;  // uniform over the workgroup
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          bf16x8 a;
          if constexpr (APF)
            a = af[u][rg][pl];
          else
            a = lda_(pl, rg, k + u * 32);
#pragma unroll
          for (int j = 0; j < NC; ++j) acc[rg][j] = mfma(a, wf[u][j], acc[rg][j]);
        }
      }
    }
  };
  // Weight batches travel one ahead of the products.  The last batch is
  // multiplied after the loop, so every trip issues the next batch
  // unconditionally and the compiler waits only for the current batch before
  // multiplying it; with the next batch's loads in a branch it waited for
  // both (16-row pass: 0.680 -> 0.671 ms, the same box).
  int k = kb;
  for (; k + 32 * U < ke; k += 32 * U) {
    bf16x8 wn[U][NC], an[APF ? U : 1][RG][NPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (APF)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int pl = 0; pl < NPL; ++pl)
            if (rg < rg_end) an[u][rg][pl] = lda_(pl, rg, k + 32 * U + u * 32);
#pragma unroll
      for (int j = 0; j < NC; ++j) wn[u][j] = ldw(j, k + 32 * U + u * 32);
    }
    multiply(k);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < NC; ++j) wf[u][j] = wn[u][j];
      if constexpr (APF)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int pl = 0; pl < NPL; ++pl) af[u][rg][pl] = an[u][rg][pl];
    }
  }
  multiply(k);

  __shared__ float rnorm[RG * 16];
  if (norm) {
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
      const int row = ks + KS * j;
      const float t = sum_wave((sqv[j][0] + sqv[j][1]) + (sqv[j][2] + sqv[j][3]));
      if (lane == 0 && row < RG * 16) rnorm[row] = 1.0f / sqrtf(t / (float)ga.ep.norm_n + ga.ep.eps);
    }
  }
  __shared__ f32x4 red[KS][RG * NC][64];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int j = 0; j < NC; ++j) red[ks][rg * NC + j][lane] = acc[rg][j];
  __syncthreads();
  if constexpr (EPI == EPI_ARGMAX || EPI == EPI_SAMPLE) {
    argmax_tail<RG, NC, KS, EPI == EPI_SAMPLE>(ga.ep, tile0, red, lane, ks);
  } else {
    for (int it = ks; it < RG * NC; it += KS) {
      if (it / NC >= rg_end) break;  // row groups this workgroup skipped: nothing to store
      f32x4 s = red[0][it][lane];
#pragma unroll
      for (int q = 1; q < KS; ++q) s += red[q][it][lane];
      if (norm) {
        const int r0 = (it / NC) * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] *= rnorm[r0 + i];
      }
      epilogue<EPI>(ga.ep, st, tile0 + it % NC, (it / NC) * 16, s, lane, kc);
    }
  }
}

// Workgroup (x, y) takes NC column tiles from tile x NC and K chunk y.
template <int EPI, int MAP, int NC, int RG, bool SPLIT, int KS = kSkinnyWaves, bool PK = false>
__global__ __launch_bounds__(KS * 64) void k_skinny(GemmArgs ga, SeqTable st) {
  skinny_body<EPI, MAP, NC, RG, SPLIT, KS, PK>(ga, st, blockIdx.x * NC, blockIdx.y, gridDim.y);
}

// q|k|v over the rows of a fused step (the block's rows, then appended
// context rows that need only K / V): the first q_groups column groups (the
// q columns) take the one-row-group body, which keeps A one batch ahead of
// the products, and the k|v groups take both row groups.  Rows 0..15 get the
// same products in the same order either way (16-row block + 16 appended
// rows: 14.3 -> about 12.8 us per layer, draft step 0.710 -> 0.702 ms, same
// box).
template <int NC, bool SPLIT, int KS, bool PK>
__global__ __launch_bounds__(KS * 64) void k_skinny_qkv_rows(GemmArgs ga, SeqTable st, int q_groups) {
  if ((int)blockIdx.x < q_groups)
    skinny_body<EPI_PARTIAL, MAP_QKV, NC, 1, SPLIT, KS, PK>(ga, st, blockIdx.x * NC, blockIdx.y, gridDim.y);
  else
    skinny_body<EPI_PARTIAL, MAP_QKV, NC, 2, SPLIT, KS, PK>(ga, st, blockIdx.x * NC, blockIdx.y, gridDim.y);
}

// ---------------------------------------------------------------------------
// Whole-K few-row GEMM (16 rows): one 16-column tile per workgroup, its K over
// kWholeKWaves waves of SPW 32-k steps each and not split across workgroups,
// so the epilogue sees finished sums.  Every weight and A fragment a wave
// needs is loaded before its first product (a scheduling barrier keeps the
// compiler from interleaving loads and products), so each CU has its whole
// share of the weights in flight at once; the waves' tiles then meet in LDS
// in a fixed order.  Weights come as tile-major packed blocks (the tile's
// K / 32 blocks of 1 KB are contiguous) or as row-major rows: the same sums
// in the same order.  The epilogue is EPI_RESID: the residual add and the
// first half of the next RMSNorm (gain * x and the per-tile sums of squares;
// the following SwiGLU GEMM applies the per-row factor), which takes the
// place of a separate reduce-and-normalise kernel after a split-K GEMM.
// ---------------------------------------------------------------------------
constexpr int kWholeKWaves = 8;

template <int SPW, bool PK>
__global__ __launch_bounds__(kWholeKWaves * 64) void k_whole_k(GemmArgs ga) {
  constexpr int W = kWholeKWaves;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x, col = tile * 16 + c, s0 = wv * SPW;
  const EpiParams& ep = ga.ep;
  // wave 0's epilogue operands (x of its four rows at this column, the gain)
  // are loaded first, so they have landed before the products
  float xv[4] = {0.f, 0.f, 0.f, 0.f}, gv = 0.f;
  if (wv == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i < ep.M) xv[i] = ep.x[(size_t)(4 * g + i) * ep.ldo + col];
    gv = bf16_val(ep.gain[col]);
  }
  const u16* wp = PK ? ga.wpack + ((size_t)tile * (ga.K / 32) * 64 + lane) * 8 + (size_t)s0 * 512
                     : ga.w.w0 + (size_t)col * ga.K + g * 8 + s0 * 32;
  const int row = min(c, ga.a_rows - 1);
  const u16* ah = ga.a_hi + (size_t)row * ga.lda + g * 8 + s0 * 32;
  const u16* al = ga.a_lo + (size_t)row * ga.lda + g * 8 + s0 * 32;
  bf16x8 wf[SPW], fh[SPW], fl[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    wf[s] = PK ? ld_frag_stream(wp + s * 512) : ld_frag(wp + s * 32);
    fh[s] = ld_frag(ah + s * 32);
    fl[s] = ld_frag(al + s * 32);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    acc = mfma(fh[s], wf[s], acc);
    acc = mfma(fl[s], wf[s], acc);
  }
  __shared__ f32x4 red[W][64];
  red[wv][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
  f32x4 v = red[0][lane];
#pragma unroll
  for (int q = 1; q < W; ++q) v += red[q][lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    float xn = 0.f;
    if (r < ep.M) {
      xn = xv[i] + v[i];
      ep.x[(size_t)r * ep.ldo + col] = xn;
      u16 h, l;
      split_pair(gv * xn, h, l);
      ep.out_hi[(size_t)r * ep.ldh + col] = h;
      ep.out_lo[(size_t)r * ep.ldh + col] = l;
    }
    const float sq = sum_row16(xn * xn);
    if (c == 0) ep.ssq[(size_t)r * ga.n_tiles + tile] = sq;
  }
}

bool gemm_whole_k_fits(int n_tiles, int K, int Mp) {
  if (Mp != 16 || n_tiles < 1 || n_tiles > 256 || n_tiles % 4 || K % (32 * kWholeKWaves)) return false;
  const int spw = K / (32 * kWholeKWaves);
  return spw == 1 || spw == 2 || spw == 4 || spw == 8 || spw == 16;
}

template <bool PK>
static hipError_t whole_k_launch(const GemmArgs& g, hipStream_t s) {
  const dim3 grid(g.n_tiles), blk(kWholeKWaves * 64);
  switch (g.K / (32 * kWholeKWaves)) {
    case 1: hipLaunchKernelGGL((k_whole_k<1, PK>), grid, blk, 0, s, g); break;
    case 2: hipLaunchKernelGGL((k_whole_k<2, PK>), grid, blk, 0, s, g); break;
    case 4: hipLaunchKernelGGL((k_whole_k<4, PK>), grid, blk, 0, s, g); break;
    case 8: hipLaunchKernelGGL((k_whole_k<8, PK>), grid, blk, 0, s, g); break;
    case 16: hipLaunchKernelGGL((k_whole_k<16, PK>), grid, blk, 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Many-row GEMM (M a multiple of 128): BM x BN output tile (BN 256, 240 or
// 192) per workgroup of BM / 64 x WN waves, each 64 rows x BN / WN columns,
// over K chunk kc of the launch's K chunks; a launch covers the column tiles
// [nt0, nt_end) of width BN (all of them, or one part of an LM head split
// into two launches).  K runs in 32-wide slabs; each
// slab (the A planes' BM rows and the BN weight rows) is copied by
// global_load_lds (16 bytes per lane, 1 KB per wave instruction) straight
// into one of S stage arrays in LDS, so S - 1 slabs are in flight without
// holding registers.  Lane l of a wave's j-th copy writes physical 16-byte
// chunk (wave IPW + j) 64 + l of the stage, i.e. chunk pc of LDS row r, and
// loads the logical chunk pc ^ ((r >> 1) & 3) of that row (big_swz).  Per
// slab: wait until this wave's copies of the slab have landed (vmcnt),
// barrier (every wave's copies landed, every wave done with the previous
// slab), issue slab kt + S - 1 into the stage slab kt - 1 used, multiply
// slab kt.  A rows past a_rows read row a_rows - 1 (an output row depends
// only on its own A row, and no epilogue consumes rows >= M); a last column
// tile past n_tiles reads a valid weight row and skips its epilogue.
// Workgroup ids are dealt round-robin over the eight XCDs; the grid is padded
// to a multiple of eight (padding workgroups exit at once) and id i takes
// logical tile (i % 8) (count / 8) + i / 8, so the row tiles that share a
// weight tile run on one XCD and share its L2 (32-sequence LM head, 1188
// tiles: 1.169 -> 1.138 ms).
// Logical tiles run over the row tiles first, then the K chunks, then the
// column tiles.  Epilogues are the per-16x16-tile ones above.
// ---------------------------------------------------------------------------

// One 16-byte-per-lane global -> LDS copy: the wave's 64 lanes fill 1 KB at
// LDS address lds (wave-uniform) + 16 lane.  Issued from asm so that the
// compiler does not wait for every outstanding copy before each LDS read;
// the kernel waits for its copies itself (wait_vmcnt) before the barrier
// that publishes a stage.  The copy takes its LDS address from m0, which the
// asm saves and restores (the compiler may keep a value there); one wait
// state separates the m0 write from the copy that reads it.
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
  const uint32_t addr = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(addr)
      : "memory");
}

// s_waitcnt with vmcnt <= N and the other counters left alone (gfx9 field
// layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr int kBigBN = 256;

// 16-byte chunk c of LDS row r (2 BK bytes per row) sits at chunk
// c ^ ((r >> 1) & (BK / 8 - 1)) of the row, which spreads the 16 rows one
// fragment read touches over the bank groups.
template <int BK>
__device__ __forceinline__ int big_swz(int row, int ch) {
  constexpr int CPR = BK / 8;  // 16-byte chunks per row
  return row * CPR + (ch ^ ((row >> 1) & (CPR - 1)));
}

template <int EPI, int MAP, bool SPLIT, int BM, int WM, int WN, int S, int BN = kBigBN>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_dl(GemmArgs ga, SeqTable st, int mt, int kcn, int nt0,
                                                          int nt_end, int slot0) {
  constexpr int BK = 32, NP = SPLIT ? 2 : 1, NW = WM * WN, CPR = BK / 8;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  static_assert(BN % (WN * 16) == 0, "whole MFMA tiles per wave");
  constexpr int ACH = BM * CPR, WCH = BN * CPR, REAL = NP * ACH + WCH;
  // copies per wave per slab; a stage that does not split into whole wave
  // copies (192-column tiles) is padded: the surplus copies repeat A chunks
  // into a pad area at the end of the stage, which nothing reads
  constexpr int IPW = (REAL + 64 * NW - 1) / (64 * NW), STAGE = IPW * 64 * NW;
  static_assert(ACH % 64 == 0 && STAGE - REAL <= ACH, "pad copies repeat A chunks");
  static_assert(S >= 2 && S <= 4, "two to four stages");
  __shared__ u32x4 st0[STAGE];
  __shared__ u32x4 st1[STAGE];
  __shared__ u32x4 st2[S > 2 ? STAGE : 1];
  __shared__ u32x4 st3[S > 3 ? STAGE : 1];
  constexpr bool AMAX = EPI == EPI_ARGMAX || EPI == EPI_SAMPLE;
  __shared__ u64 rk[AMAX ? BM : 1];  // LM head: per-row key of the workgroup's columns

  const int nwg = gridDim.x;
  const int bid = (nwg & 7) == 0 ? (int)(blockIdx.x & 7) * (nwg >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int m_t = bid % mt, kc = (bid / mt) % kcn, n_t = nt0 + bid / (mt * kcn);
  if (n_t >= nt_end) return;  // grid padding to whole rounds of eight XCDs
  if constexpr (AMAX) {
    for (int i = threadIdx.x; i < BM; i += WM * WN * 64) rk[i] = 0;
    __syncthreads();
  }
  const int row0 = m_t * BM, tile0 = n_t * (BN / 16);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const int K = ga.K, kspan = K / kcn, kbase = kc * kspan;

  const u16* gp[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int pp = (wave * IPW + j) * 64 + lane;  // physical chunk of the stage
    const int p = pp < REAL ? pp : pp - REAL;      // a pad copy loads an A chunk again
    const int plane = p / ACH;                     // 0 .. NP-1: A planes; NP: weights
    const int q = p - (plane < NP ? plane : NP) * ACH;
    const int r = q / CPR, lc = (q % CPR) ^ ((r >> 1) & (CPR - 1));
    if (plane < NP) {
      const int arow = min(row0 + r, ga.a_rows - 1);
      gp[j] = (plane == 0 ? ga.a_hi : ga.a_lo) + (size_t)arow * ga.lda + kbase + lc * 8;
    } else {
      const int tile = min(tile0 + (r >> 4), ga.n_tiles - 1);
      gp[j] = weight_row<MAP>(ga.w, ga.ep, tile, r & 15, K) + kbase + lc * 8;
    }
  }
  u32x4* const stg[4] = {st0, st1, st2, st3};
  auto issue = [&](u32x4* sp, int k0) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) dma16(gp[j] + k0, sp + (wave * IPW + j) * 64);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4* Sm) {
    bf16x8 wf[TN];
#pragma unroll
    for (int ct = 0; ct < TN; ++ct)
      wf[ct] = __builtin_bit_cast(bf16x8, Sm[NP * ACH + big_swz<BK>(wn * TN * 16 + ct * 16 + c, g)]);
#pragma unroll
    for (int rg = 0; rg < TM; ++rg)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, Sm[p * ACH + big_swz<BK>(wm * TM * 16 + rg * 16 + c, g)]);
#pragma unroll
        for (int ct = 0; ct < TN; ++ct) acc[rg][ct] = mfma(a, wf[ct], acc[rg][ct]);
      }
  };

  const int nk = kspan / BK;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(stg[s], s * BK);
  for (int kt0 = 0; kt0 < nk; kt0 += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kt = kt0 + s;
      if (kt < nk) {
        // slab kt landed: the copies of the slabs issued after it may stay
        // in flight (S - 2 of them while any remain to be issued)
        if (kt + S - 2 < nk)
          wait_vmcnt<(S - 2) * IPW>();
        else
          wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + S - 1 < nk) issue(stg[(s + S - 1) % S], (kt + S - 1) * BK);
        compute(stg[s]);
      }
    }
  }
  if constexpr (AMAX) {
    // one key per row for the workgroup's 256 columns: the wave's tiles are
    // combined in registers, the waves that share rows through LDS
#pragma unroll
    for (int rg = 0; rg < TM; ++rg) {
      const int r0 = row0 + wm * TM * 16 + rg * 16;
      u64 best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
      for (int ct = 0; ct < TN; ++ct) {
        const int tile = tile0 + wn * TN + ct;
        if (tile >= ga.n_tiles) break;  // uniform over the wave
        u64 key[4];
        argmax_tile_keys<EPI == EPI_SAMPLE>(ga.ep, tile, r0, acc[rg][ct], lane, key);
#pragma unroll
        for (int i = 0; i < 4; ++i) best[i] = key[i] > best[i] ? key[i] : best[i];
      }
      if (c == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (best[i]) atomicMax(&rk[r0 - row0 + 4 * g + i], best[i]);
      }
    }
    __syncthreads();
    const size_t slot = (size_t)(slot0 + n_t - nt0);  // this column tile's partial keys
    for (int i = threadIdx.x; i < BM; i += WM * WN * 64)
      if (row0 + i < ga.ep.Mp) ga.ep.amax_part[slot * ga.ep.Mp + row0 + i] = rk[i];
  } else {
#pragma unroll
    for (int ct = 0; ct < TN; ++ct) {
      const int tile = tile0 + wn * TN + ct;
      if (tile >= ga.n_tiles) break;  // uniform over the wave
#pragma unroll
      for (int rg = 0; rg < TM; ++rg)
        epilogue<EPI>(ga.ep, st, tile, row0 + wm * TM * 16 + rg * 16, acc[rg][ct], lane, kc);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention over [injected context | block] keys.
//
// One workgroup per (sequence, kv head, key split), or with anchored blocks
// that share a context per (group of blocks, kv head, key split).  Its waves
// are the query units that read this kv head: (HPW q heads of the GQA group)
// x (16-row query tile) x (block of the group); at least four waves are
// launched so that a cache tile is staged by enough threads (surplus waves
// only stage).  A group's blocks are sorted by anchor; its context tiles
// are those of its longest prefix, and a wave skips tiles past its own
// block's prefix.  Each K / V fragment a wave reads from LDS feeds all HPW
// of its heads.  Scores are taken in base-2 units (scaled by
// scale log2(e), so the running max is too) and each softmax weight is one
// fma and one hardware base-2 exponential.  Each 64-key cache tile is
// copied once from HBM (contiguous, prefetched into registers while the
// previous tile is used) into LDS, where every query unit of the group reads
// it.  Per 32-key half a wave computes S^T = K Q^T with keys as MFMA rows, so
// that the probabilities land in the register layout the P.V product takes as
// its B operand, keeps a running max / sum per query row (online softmax) and
// accumulates O^T = V^T P^T from the transposed V planes.  MFMA row rho of
// key tile kt (0 or 1) is key 8 (rho / 4) + 4 kt + rho % 4 of the half, so
// lane group q ends up holding keys 8q .. 8q+7 — exactly one B fragment.
// fp32 x fp32 products are taken as hi*hi + hi*lo + lo*hi.
// The keys are either [context | block] in the cache, or (anchored blocks
// that share a context) the context prefix in the cache followed by one
// tile of the block's own keys kept apart in the workspace (for a group:
// one such tile per member, after the shared context tiles).
// With one split the result is normalised and written directly; otherwise
// partial (m, l, O) go to a workspace and the merge kernel combines them in
// split order.
// ---------------------------------------------------------------------------

// 16-byte chunk swizzles of the LDS copy of a tile (bijections within a row):
// the 16 keys one K fragment read touches, and the 16 V^T rows one V fragment
// read touches, fall in distinct bank groups.
__device__ __forceinline__ int k_swz(int key) { return (((key >> 3) & 3) << 2) | (key & 3); }
__device__ __forceinline__ int v_swz(int drow) { return (drow >> 1) & 7; }

template <int D>
__device__ __forceinline__ int lds_chunk(int cidx) {
  constexpr int CH = D / 8, PL = kTileKeys * CH;  // chunks per K row, per plane
  const int plane = cidx / PL, w = cidx % PL;
  if (plane < 2) {
    const int key = w / CH, ch = w % CH;
    return plane * PL + key * CH + (ch ^ (k_swz(key) & (CH - 1)));
  }
  const int drow = w / 8, ch = w % 8;
  return plane * PL + drow * 8 + (ch ^ v_swz(drow));
}

template <int D, int NW, bool GRP, int HPW, bool HV>
__global__ __launch_bounds__(NW * 64) void k_attn_tiles(const u16* __restrict__ q_hi,
                                                         const u16* __restrict__ q_lo,
                                                         const u16* __restrict__ kv, int64_t kv_tiles,
                                                         const u16* __restrict__ bkv, int bkv_tiles,
                                                         float* __restrict__ part_o,
                                                         float* __restrict__ part_ml,
                                                         u16* __restrict__ o_hi, u16* __restrict__ o_lo,
                                                         int block, int n_q, int n_kv, int splits,
                                                         float scale, SeqTable st,
                                                         std::conditional_t<GRP, AttnGroups, int> grp) {
  constexpr int CH = D / 8, PL = kTileKeys * CH;
  constexpr int TILE_CH = 4 * PL;  // 16-byte chunks per cache tile
  constexpr int NT = NW * 64;
  constexpr int CPT = TILE_CH / NT;
  static_assert(TILE_CH % NT == 0, "tile must split evenly over the threads");
  constexpr int DS = D / 32, DT = D / 16;
  const float su = scale * 1.4426950408889634f;  // scale log2(e): scores to base-2 units
  __shared__ u32x4 lds[TILE_CH];

  // grid (kv head x split, unit).  The unit index comes straight from the
  // launch, so its table entries are read together with the other kernel
  // arguments: the prologue waits for argument memory once, not once per
  // dependent lookup.  The wave index is the same on every lane of a wave,
  // which keeps the per-wave lookups scalar.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int unit = blockIdx.y;  // the block, or the group of blocks
  int u_pos = 0, u_row = 0, u_slot = 0;
  if constexpr (!GRP) {
    u_pos = st.pos_base[unit];
    u_row = st.row_start[unit];
    u_slot = st.slot_base[unit];
  }
  const int s = blockIdx.x % splits, gkv = blockIdx.x / splits;
  const int G = n_q / n_kv, HG = G / HPW, qtiles = (block + 15) / 16, upb = HG * qtiles;
  // HV (one block per unit): waves upb .. 2 upb - 1 take the second 32 keys
  // of every tile for the same query units, and the two halves' (m, l, O)
  // are combined at the end
  static_assert(!(HV && GRP), "halves are for one-block units");
  const int half = HV ? wave / upb : 0;
  const int mj = HV ? (half < 2 ? 0 : 1) : wave / upb, wu = wave % upb;  // member mj, query unit wu
  int nb = 1, b0 = unit, b = mj == 0 ? unit : -1;
  if constexpr (GRP) {
    nb = 0;
#pragma unroll
    for (int j = 0; j < kAttnGroup; ++j) nb += grp.member[unit][j] >= 0;
    b0 = grp.member[unit][0];
    b = mj < kAttnGroup ? grp.member[unit][mj] : -1;
  }
  const bool comp = b >= 0;
  const int h0 = gkv * G + (wu % HG) * HPW, qt = wu / HG;  // this wave's heads h0 .. h0 + HPW - 1

  // context tiles in the cache (with the block's keys when they sit there),
  // shared by the unit's blocks, then with a separate block area one tile
  // of each member's own keys
  const bool sep = bkv != nullptr;
  int maxct = 0;
  if constexpr (GRP) {
    for (int j = 0; j < nb; ++j)
      maxct = max(maxct, (st.pos_base[grp.member[unit][j]] + kTileKeys - 1) / kTileKeys);
  } else {
    maxct = (u_pos + (sep ? 0 : block) + kTileKeys - 1) / kTileKeys;
  }
  // one-block units: b is the unit whenever comp holds
  const int n_keys = comp ? (GRP ? st.pos_base[b] : u_pos) + (sep ? 0 : block) : 0;
  const int ntile = maxct + (sep ? nb : 0);
  const int tps = (ntile + splits - 1) / splits;
  const int t0 = s * tps, t1 = min(ntile, t0 + tps);
  const u32x4* src = reinterpret_cast<const u32x4*>(
      kv + kv_tile_offset(gkv, (GRP ? st.slot_base[b0] : u_slot) / kTileKeys, kv_tiles, D));
  auto tile_ptr = [&](int t) -> const u32x4* {
    if (t < maxct) return src + (size_t)t * TILE_CH;
    int mb = unit;
    if constexpr (GRP) mb = grp.member[unit][t - maxct];
    return reinterpret_cast<const u32x4*>(bkv + kv_tile_offset(gkv, mb, bkv_tiles, D));
  };

  // the first tile's loads go out before q's: the tile is needed first
  u32x4 stage[CPT];
  if (t0 < t1) {
    const u32x4* tp = tile_ptr(t0);
#pragma unroll
    for (int j = 0; j < CPT; ++j) stage[j] = HV ? ld_tile_stream(tp + tid + j * NT) : tp[tid + j * NT];
  }

  const int qi = qt * 16 + c;
  const bool qvalid = comp && qi < block;
  const size_t qrow = (size_t)((GRP ? st.row_start[comp ? b : b0] : u_row) + qi);
  bf16x8 qh[HPW][DS], ql[HPW][DS];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const size_t qoff = qrow * (n_q * D) + (h0 + hh) * D + g * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qh[hh][ds] = qvalid ? ld_frag(q_hi + qoff + ds * 32) : zero_frag();
      ql[hh][ds] = qvalid ? ld_frag(q_lo + qoff + ds * 32) : zero_frag();
    }
  }
  f32x4 o[HPW][DT];
  float m[HPW], l[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[hh][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[hh] = -INFINITY;
    l[hh] = 0.f;
  }
  for (int t = t0; t < t1; ++t) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) lds[lds_chunk<D>(tid + j * NT)] = stage[j];
    __syncthreads();
    if (t + 1 < t1) {
      const u32x4* tp = tile_ptr(t + 1);
#pragma unroll
      for (int j = 0; j < CPT; ++j) stage[j] = HV ? ld_tile_stream(tp + tid + j * NT) : tp[tid + j * NT];
    }
    if (!comp) continue;
    // valid keys of this tile for this wave's block (none: the tile belongs
    // to a longer member's prefix or is another member's block tile)
    const int lim = t < maxct ? n_keys - t * kTileKeys : (t - maxct == mj ? block : 0);
    if (lim <= (HV ? half * 32 : 0)) continue;  // no valid key for this wave (uniform over the wave)

    // every K fragment read from LDS serves all HPW heads of the wave.  A
    // wave covers NHF 32-key halves of the tile: both, or with HV only its
    // own (half), so that it neither scores nor exponentiates the other
    // half's keys
    constexpr int NHF = HV ? 1 : 2;
    f32x4 sacc[HPW][NHF][2];
#pragma unroll
    for (int h2 = 0; h2 < NHF; ++h2)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int hf = HV ? half : h2;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) sacc[hh][h2][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int key = hf * 32 + 8 * (c >> 2) + 4 * kt + (c & 3);
        const int sw = k_swz(key) & (CH - 1);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const int ch = (ds * 4 + g) ^ sw;
          const bf16x8 kh = __builtin_bit_cast(bf16x8, lds[key * CH + ch]);
          const bf16x8 kl = __builtin_bit_cast(bf16x8, lds[PL + key * CH + ch]);
#pragma unroll
          for (int hh = 0; hh < HPW; ++hh) {
            sacc[hh][h2][kt] = mfma(kh, qh[hh][ds], sacc[hh][h2][kt]);
            sacc[hh][h2][kt] = mfma(kh, ql[hh][ds], sacc[hh][h2][kt]);
            sacc[hh][h2][kt] = mfma(kl, qh[hh][ds], sacc[hh][h2][kt]);
          }
        }
      }
    // keys past lim are masked; a tile whose keys are all valid for this
    // wave skips the comparisons (uniform over the wave).  The running max m
    // is kept in base-2 units of the scaled score, u = s scale log2(e), so
    // that each weight is one fma and one exp2
    const bool full = lim >= (HV ? (half + 1) * 32 : kTileKeys);
    float p[HPW][NHF * 8];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float sv[NHF * 8];
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int j = 0; j < NHF * 8; ++j) {
          sv[j] = sacc[hh][j / 8][(j / 4) & 1][j & 3];
          mx = fmaxf(mx, sv[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NHF * 8; ++j) {
          const int key = (HV ? half : j / 8) * 32 + 8 * g + 4 * ((j / 4) & 1) + (j & 3);
          sv[j] = key < lim ? sacc[hh][j / 8][(j / 4) & 1][j & 3] : -INFINITY;
          mx = fmaxf(mx, sv[j]);
        }
      }
      mx = max_xor<32>(max_xor<16>(mx));
      const float m_new = fmaxf(m[hh], mx * su);  // su > 0: the max of the scaled scores
      const float corr = fast_exp2(m[hh] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < NHF * 8; ++j) {
        p[hh][j] = fast_exp2(fmaf(sv[j], su, -m_new));
        ps += p[hh][j];
      }
      ps = sum_xor<32>(sum_xor<16>(ps));
      l[hh] = l[hh] * corr + ps;
      m[hh] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[hh][dt] *= corr;
    }
#pragma unroll
    for (int h2 = 0; h2 < NHF; ++h2) {
      const int hf = HV ? half : h2;
      bf16x8 ph[HPW], pl[HPW];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) split_frag(p[hh] + h2 * 8, ph[hh], pl[hh]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int drow = dt * 16 + c;
        const int ch = (hf * 4 + g) ^ v_swz(drow);
        const bf16x8 vh = __builtin_bit_cast(bf16x8, lds[2 * PL + drow * 8 + ch]);
        const bf16x8 vl = __builtin_bit_cast(bf16x8, lds[3 * PL + drow * 8 + ch]);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          o[hh][dt] = mfma(vh, ph[hh], o[hh][dt]);
          o[hh][dt] = mfma(vh, pl[hh], o[hh][dt]);
          o[hh][dt] = mfma(vl, ph[hh], o[hh][dt]);
        }
      }
    }
  }
  if constexpr (HV) {
    // the second half's waves hand (m, l, O) to the first half's through
    // the tile buffer; weights 2^(m_half - max) as in the online softmax
    float* xo = reinterpret_cast<float*>(lds) + (size_t)wu * (DT * 4 + 2) * 64;
    __syncthreads();  // every wave is done with the last tile
    if (comp && half == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) xo[(dt * 4 + i) * 64 + lane] = o[0][dt][i];
      xo[DT * 4 * 64 + lane] = m[0];
      xo[(DT * 4 + 1) * 64 + lane] = l[0];
    }
    __syncthreads();
    if (!comp || half != 0) return;
    const float m1 = xo[DT * 4 * 64 + lane], l1 = xo[(DT * 4 + 1) * 64 + lane];
    const float M = fmaxf(m[0], m1);
    if (M != -INFINITY) {
      const float w0 = fast_exp2(m[0] - M), w1 = fast_exp2(m1 - M);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[0][dt][i] = o[0][dt][i] * w0 + xo[(dt * 4 + i) * 64 + lane] * w1;
      l[0] = l[0] * w0 + l1 * w1;
      m[0] = M;
    }
  }
  if (!comp) return;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = h0 + hh;
    if (splits == 1) {
      if (!qvalid) continue;
      const float inv = 1.0f / l[hh];
      const size_t ob = qrow * (n_q * D) + h * D + g * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u16 hv, lv;
          split_pair(o[hh][dt][i] * inv, hv, lv);
          o_hi[ob + dt * 16 + i] = hv;
          o_lo[ob + dt * 16 + i] = lv;
        }
      continue;
    }
    const size_t pidx = ((size_t)(b * n_q + h) * qtiles + qt) * splits + s;
    float* po = part_o + pidx * 16 * D + c * D + g * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[hh][dt];
    if (g == 0) {
      part_ml[pidx * 32 + c] = m[hh];
      part_ml[pidx * 32 + 16 + c] = l[hh];
    }
  }
}

// The same attention for one-block units with at most four query units (q
// heads of the GQA group x 16-row query tiles), with two waves per query
// unit (one per 32-key half of every tile), for splits of a few tiles.
// Roles are split and the tile buffer doubled, so that one barrier per tile
// suffices and the copy into LDS leaves the critical path: waves 8 .. 15
// only stage (each holding an eighth of the next tile in registers) and
// write tile t + 1 into one LDS buffer while the computing waves read tile t
// from the other.  A computing wave reads the K (V) fragments of the next
// k-step (d tile) before multiplying the current ones.  Every product and sum
// is the one k_attn_tiles forms, in the same order, and the two give bitwise
// equal results (checked at 1 to 26 splits, 4096 to 8192 keys, 8 and 32
// sequences).  8192 keys in 26 splits of five tiles: 20.3 -> 18.7 us per
// layer; 4096 keys, 13 splits: 16.1 -> 13.8 us; with 33-tile splits, 32 x
// 2048, it measured 3% slower, so those keep k_attn_tiles.
template <int D>
__global__ __launch_bounds__(1024) void k_attn_staged(const u16* __restrict__ q_hi, const u16* __restrict__ q_lo,
                                                      const u16* __restrict__ kv, int64_t kv_tiles,
                                                      float* __restrict__ part_o, float* __restrict__ part_ml,
                                                      u16* __restrict__ o_hi, u16* __restrict__ o_lo, int block,
                                                      int n_q, int n_kv, int splits, float scale, SeqTable st) {
  constexpr int CH = D / 8, PL = kTileKeys * CH, TILE_CH = 4 * PL;
  constexpr int NS = 512, CPS = TILE_CH / NS;  // staging threads, 16-byte chunks of a tile per staging thread
  constexpr int DS = D / 32, DT = D / 16;
  const float su = scale * 1.4426950408889634f;  // scale log2(e): scores to base-2 units
  __shared__ u32x4 ldsb[2 * TILE_CH];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int unit = blockIdx.y;
  const int u_pos = st.pos_base[unit], u_row = st.row_start[unit], u_slot = st.slot_base[unit];
  const int s = blockIdx.x % splits, gkv = blockIdx.x / splits;
  const int G = n_q / n_kv, qtiles = (block + 15) / 16, upb = G * qtiles;
  const bool stager = wave >= 8;
  const int half = wave / upb, wu = wave % upb;
  const bool comp = !stager && wave < 2 * upb;
  const int h = gkv * G + wu % G, qt = wu / G;
  const int n_keys = u_pos + block;
  const int ntile = (n_keys + kTileKeys - 1) / kTileKeys;
  const int tps = (ntile + splits - 1) / splits;
  const int t0 = s * tps, t1 = min(ntile, t0 + tps);
  const u32x4* src = reinterpret_cast<const u32x4*>(kv + kv_tile_offset(gkv, u_slot / kTileKeys, kv_tiles, D));

  if (stager) {
    // Loads are issued unconditionally (past the split's last tile they
    // re-read it from L2), which keeps the compiler's wait before each LDS
    // write to exactly the loads of the tile being written.  Barriers match
    // the computing waves' one for one.
    const int sid = tid - NS;
    const int tl = max(t1 - 1, 0);
    auto tile_src = [&](int t) { return src + (size_t)min(t, tl) * TILE_CH + sid; };
    u32x4 sa[CPS];
    const u32x4* pa = tile_src(t0);
#pragma unroll
    for (int j = 0; j < CPS; ++j) sa[j] = ld_tile_stream(pa + j * NS);
    if (t0 < t1) {
#pragma unroll
      for (int j = 0; j < CPS; ++j) ldsb[lds_chunk<D>(sid + j * NS)] = sa[j];
      pa = tile_src(t0 + 1);
#pragma unroll
      for (int j = 0; j < CPS; ++j) sa[j] = ld_tile_stream(pa + j * NS);
    }
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
      if (t + 1 < t1) {
        u32x4* dst = ldsb + ((t - t0 + 1) & 1) * TILE_CH;
#pragma unroll
        for (int j = 0; j < CPS; ++j) dst[lds_chunk<D>(sid + j * NS)] = sa[j];
        pa = tile_src(t + 2);
#pragma unroll
        for (int j = 0; j < CPS; ++j) sa[j] = ld_tile_stream(pa + j * NS);
      }
      __syncthreads();
    }
    __syncthreads();  // the two barriers of the halves' combine
    __syncthreads();
    return;
  }

  const int qi = qt * 16 + c;
  const bool qvalid = comp && qi < block;
  const size_t qrow = (size_t)(u_row + qi);
  bf16x8 qh[DS], ql[DS];
  {
    const size_t qoff = qrow * (n_q * D) + h * D + g * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qh[ds] = qvalid ? ld_frag(q_hi + qoff + ds * 32) : zero_frag();
      ql[ds] = qvalid ? ld_frag(q_lo + qoff + ds * 32) : zero_frag();
    }
  }
  f32x4 o[DT];
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // MFMA row rho of 16-key tile kt is key 8 (rho / 4) + 4 kt + rho % 4 of
  // the half, as in k_attn_tiles; both tiles are scored together
  const int key0 = half * 32 + 8 * (c >> 2) + (c & 3), key1 = key0 + 4;
  const int sw0 = k_swz(key0) & (CH - 1), sw1 = k_swz(key1) & (CH - 1);
  auto tile = [&](const u32x4* lds, int t) {
    const int lim = n_keys - t * kTileKeys;  // valid keys of the tile
    if (lim <= half * 32) return;            // none in this wave's half (uniform)
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    bf16x8 kf[2][4];
    auto kld = [&](bf16x8* f, int ds) {
      f[0] = __builtin_bit_cast(bf16x8, lds[key0 * CH + ((ds * 4 + g) ^ sw0)]);
      f[1] = __builtin_bit_cast(bf16x8, lds[PL + key0 * CH + ((ds * 4 + g) ^ sw0)]);
      f[2] = __builtin_bit_cast(bf16x8, lds[key1 * CH + ((ds * 4 + g) ^ sw1)]);
      f[3] = __builtin_bit_cast(bf16x8, lds[PL + key1 * CH + ((ds * 4 + g) ^ sw1)]);
    };
    kld(kf[0], 0);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      if (ds + 1 < DS) kld(kf[(ds + 1) & 1], ds + 1);
      __builtin_amdgcn_sched_barrier(0);  // keep the next k-step's reads ahead of these products
      const bf16x8* f = kf[ds & 1];
      sacc[0] = mfma(f[0], qh[ds], sacc[0]);
      sacc[1] = mfma(f[2], qh[ds], sacc[1]);
      sacc[0] = mfma(f[0], ql[ds], sacc[0]);
      sacc[1] = mfma(f[2], ql[ds], sacc[1]);
      sacc[0] = mfma(f[1], qh[ds], sacc[0]);
      sacc[1] = mfma(f[3], qh[ds], sacc[1]);
    }
    // the online softmax of k_attn_tiles, m in base-2 units of the scaled score
    const bool full = lim >= (half + 1) * 32;
    float p[8], sv[8];
    float mx = -INFINITY;
    if (full) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sv[j] = sacc[j / 4][j & 3];
        mx = fmaxf(mx, sv[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = half * 32 + 8 * g + j;
        sv[j] = key < lim ? sacc[j / 4][j & 3] : -INFINITY;
        mx = fmaxf(mx, sv[j]);
      }
    }
    mx = max_xor<32>(max_xor<16>(mx));
    const float m_new = fmaxf(m, mx * su);
    const float corr = fast_exp2(m - m_new);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = fast_exp2(fmaf(sv[j], su, -m_new));
      ps += p[j];
    }
    ps = sum_xor<32>(sum_xor<16>(ps));
    l = l * corr + ps;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
    bf16x8 ph, pl;
    split_frag(p, ph, pl);
    bf16x8 vf[2][2];
    auto vld = [&](bf16x8* f, int dt) {
      const int drow = dt * 16 + c;
      const int ch = (half * 4 + g) ^ v_swz(drow);
      f[0] = __builtin_bit_cast(bf16x8, lds[2 * PL + drow * 8 + ch]);
      f[1] = __builtin_bit_cast(bf16x8, lds[3 * PL + drow * 8 + ch]);
    };
    vld(vf[0], 0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (dt + 1 < DT) vld(vf[(dt + 1) & 1], dt + 1);
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8* f = vf[dt & 1];
      o[dt] = mfma(f[0], ph, o[dt]);
      o[dt] = mfma(f[0], pl, o[dt]);
      o[dt] = mfma(f[1], ph, o[dt]);
    }
  };
  __syncthreads();  // tile t0 staged
  for (int t = t0; t < t1; ++t) {
    if (comp) tile(ldsb + ((t - t0) & 1) * TILE_CH, t);
    __syncthreads();  // tile t used; tile t + 1 staged
  }

  // the second half's waves hand (m, l, O) to the first half's through LDS
  float* xo = reinterpret_cast<float*>(ldsb) + (size_t)wu * (DT * 4 + 2) * 64;
  __syncthreads();
  if (comp && half == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) xo[(dt * 4 + i) * 64 + lane] = o[dt][i];
    xo[DT * 4 * 64 + lane] = m;
    xo[(DT * 4 + 1) * 64 + lane] = l;
  }
  __syncthreads();
  if (!comp || half != 0) return;
  const float m1 = xo[DT * 4 * 64 + lane], l1 = xo[(DT * 4 + 1) * 64 + lane];
  const float M = fmaxf(m, m1);
  if (M != -INFINITY) {
    const float w0 = fast_exp2(m - M), w1 = fast_exp2(m1 - M);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[dt][i] = o[dt][i] * w0 + xo[(dt * 4 + i) * 64 + lane] * w1;
    l = l * w0 + l1 * w1;
    m = M;
  }
  if (splits == 1) {
    if (!qvalid) return;
    const float inv = 1.0f / l;
    const size_t ob = qrow * (n_q * D) + h * D + g * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u16 hv, lv;
        split_pair(o[dt][i] * inv, hv, lv);
        o_hi[ob + dt * 16 + i] = hv;
        o_lo[ob + dt * 16 + i] = lv;
      }
    return;
  }
  const size_t pidx = ((size_t)(unit * n_q + h) * qtiles + qt) * splits + s;
  float* po = part_o + pidx * 16 * D + c * D + g * 4;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16) = o[dt];
  if (g == 0) {
    part_ml[pidx * 32 + c] = m;
    part_ml[pidx * 32 + 16 + c] = l;
  }
}

// Combine the key splits of each (sequence, q head, 16-row query tile) unit.
// Workgroup = unit x 4-row quad; wave w owns one query row: lane s reads
// split s's (m, l) while every lane loads its D/64 output columns of all
// splits (PF >= splits, from a few fixed sizes); the wave forms the
// log-sum-exp weights 2^(m_s - max) / sum_s l_s 2^(m_s - max) (the maxima
// are in base-2 units; lane s holds split s's), then each lane sums its columns over the splits in split
// order and writes the hi/lo planes [row][n_q * D].
template <int D, int PF>
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    u16* __restrict__ o_hi, u16* __restrict__ o_lo,
                                                    int block, int n_q, int splits, SeqTable st) {
  constexpr int PER = D / 64;  // PF: splits whose outputs are loaded with (m, l)
  // grid (query tile x head x quad, sequence): the sequence's first row is
  // read with the other arguments, not after them
  const int b = blockIdx.y, b_row = st.row_start[b];
  const int qtiles = (block + 15) / 16;
  const int quad = blockIdx.x & 3, uh = blockIdx.x >> 2;  // uh = h * qtiles + qt
  const int qt = uh % qtiles, h = uh / qtiles, unit = b * n_q * qtiles + uh;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = quad * 4 + wv, qi = qt * 16 + row;
  if (qi >= block) return;  // wave-uniform; the wave owns its row alone
  const size_t p0 = (size_t)unit * splits;
  const float* po = part_o + (p0 * 16 + row) * D + lane * PER;
  float m = -INFINITY, l = 0.f;
  if (lane < splits) {
    m = part_ml[(p0 + lane) * 32 + row];
    l = part_ml[(p0 + lane) * 32 + 16 + row];
  }
  float pre[PF][PER];
#pragma unroll
  for (int s = 0; s < PF; ++s)
#pragma unroll
    for (int p = 0; p < PER; ++p) pre[s][p] = s < splits ? po[(size_t)s * 16 * D + p] : 0.f;
  const float M = max_wave(m);
  const float e = lane < splits ? fast_exp2(m - M) : 0.f;  // m in base-2 units
  const float L = sum_wave(e * l);
  const float w = e / L;  // lane s: the weight of split s; read by every lane with readlane
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
  // (no early exit here: a conditional use lets the compiler sink the loads
  // above into this loop, one round trip per split)
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
#pragma unroll
    for (int p = 0; p < PER; ++p) acc[p] += s < splits ? ws * pre[s][p] : 0.f;
  }
  for (int s = PF; s < splits; ++s) {  // splits beyond the prefetched ones (none as launched)
    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
#pragma unroll
    for (int p = 0; p < PER; ++p) acc[p] += ws * po[(size_t)s * 16 * D + p];
  }
  const size_t o = (size_t)(b_row + qi) * (n_q * D) + h * D + lane * PER;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    u16 hv, lv;
    split_pair(acc[p], hv, lv);
    o_hi[o + p] = hv;
    o_lo[o + p] = lv;
  }
}

// ---------------------------------------------------------------------------
// small kernels
// ---------------------------------------------------------------------------

// One workgroup of 1024 threads per row.  x[row] = E[token] (embedding
// mode) or x[row] += sum_{q < kc} part[q][row] (residual mode, fixed order),
// then the RMSNorm of the new x row, gain * x / sqrt(mean(x^2) + eps), is
// written as hi/lo planes.  Thread t owns the NV 4-element chunks t + 1024 v
// of the row: every load it needs (x, all chunk partials, the gains) is
// issued at once, and the new x stays in registers for the norm, so the
// kernel waits on memory once before its one workgroup reduction.  Rows
// M..Mp-1 of the planes are zero.
template <int NV>
__global__ __launch_bounds__(1024) void k_resid_norm(float* __restrict__ x, const float* __restrict__ part,
                                                     int kc, int part_rows, const int32_t* __restrict__ anchors,
                                                     const int32_t* __restrict__ block_tokens,
                                                     const u16* __restrict__ E, int block, int mask_id, int vocab,
                                                     const u16* __restrict__ gain, u16* __restrict__ out_hi,
                                                     u16* __restrict__ out_lo, int H, int M, float eps) {
  const int row = blockIdx.x, tid = threadIdx.x;
  u16* oh = out_hi + (size_t)row * H;
  u16* ol = out_lo + (size_t)row * H;
  if (row >= M && E && part) {
    // appended rows: their fused features, summed over the K chunks in order
    const int r = row - M;
    for (int j = tid * 4; j < H; j += 4096) {
      f32x4 p[kMaxKc];
#pragma unroll
      for (int q = 0; q < kMaxKc; ++q)
        if (q < kc) p[q] = *reinterpret_cast<const f32x4*>(part + ((size_t)q * part_rows + r) * H + j);
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < kMaxKc; ++q)
        if (q < kc) v += p[q];
      u16 hh[4], ll[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split_pair(v[i], hh[i], ll[i]);
      *reinterpret_cast<uint2*>(oh + j) =
          make_uint2((uint32_t)hh[0] | ((uint32_t)hh[1] << 16), (uint32_t)hh[2] | ((uint32_t)hh[3] << 16));
      *reinterpret_cast<uint2*>(ol + j) =
          make_uint2((uint32_t)ll[0] | ((uint32_t)ll[1] << 16), (uint32_t)ll[2] | ((uint32_t)ll[3] << 16));
    }
    return;
  }
  if (row >= M) {
    for (int j = tid * 4; j < H; j += 4096) {
      *reinterpret_cast<uint2*>(oh + j) = make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(ol + j) = make_uint2(0u, 0u);
    }
    return;
  }
  float* xr = x + (size_t)row * H;
  const u16* er = nullptr;
  if (E) {
    const int b = row / block, i = row % block;
    int tok = i == 0 ? anchors[b] : (block_tokens ? block_tokens[b * (block - 1) + i - 1] : mask_id);
    tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);
    er = E + (size_t)tok * H;
  }
  f32x4 xv[NV];
  uint2 gw[NV];
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int j = tid * 4 + v * 4096;
    xv[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    gw[v] = make_uint2(0u, 0u);
    if (j >= H) continue;
    gw[v] = *reinterpret_cast<const uint2*>(gain + j);
    if (er) {
      const uint2 w = *reinterpret_cast<const uint2*>(er + j);
      xv[v] = f32x4{bf16_val(w.x & 0xFFFFu), bf16_val(w.x >> 16), bf16_val(w.y & 0xFFFFu), bf16_val(w.y >> 16)};
    } else {
      f32x4 p[kMaxKc];
#pragma unroll
      for (int q = 0; q < kMaxKc; ++q)
        if (q < kc) p[q] = *reinterpret_cast<const f32x4*>(part + ((size_t)q * part_rows + row) * H + j);
      f32x4 t = *reinterpret_cast<const f32x4*>(xr + j);
#pragma unroll
      for (int q = 0; q < kMaxKc; ++q)
        if (q < kc) t += p[q];
      xv[v] = t;
    }
    *reinterpret_cast<f32x4*>(xr + j) = xv[v];
    ss += xv[v][0] * xv[v][0] + xv[v][1] * xv[v][1] + xv[v][2] * xv[v][2] + xv[v][3] * xv[v][3];
  }
  ss = sum_wave(ss);
  __shared__ float wsum[16];
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) tot += wsum[w];
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int j = tid * 4 + v * 4096;
    if (j >= H) continue;
    const float gs[4] = {bf16_val(gw[v].x & 0xFFFFu), bf16_val(gw[v].x >> 16), bf16_val(gw[v].y & 0xFFFFu),
                         bf16_val(gw[v].y >> 16)};
    u16 hh[4], ll[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_pair(gs[i] * xv[v][i] * r, hh[i], ll[i]);
    *reinterpret_cast<uint2*>(oh + j) =
        make_uint2((uint32_t)hh[0] | ((uint32_t)hh[1] << 16), (uint32_t)hh[2] | ((uint32_t)hh[3] << 16));
    *reinterpret_cast<uint2*>(ol + j) =
        make_uint2((uint32_t)ll[0] | ((uint32_t)ll[1] << 16), (uint32_t)ll[2] | ((uint32_t)ll[3] << 16));
  }
}

// out[row][j] = hi/lo(sum_{q < kc} part[q][row][j]); rows M..out_rows-1 are zero.
__global__ __launch_bounds__(256) void k_reduce_split(const float* __restrict__ part, int kc, int part_rows, int N,
                                                      u16* __restrict__ out_hi, u16* __restrict__ out_lo, int M,
                                                      int out_rows) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)out_rows * N) return;
  const int row = (int)(idx / N);
  u16 h = 0, l = 0;
  if (row < M) {
    float s = 0.f;
    for (int q = 0; q < kc; ++q) s += part[(size_t)q * part_rows * N + idx];
    split_pair(s, h, l);
  }
  out_hi[idx] = h;
  out_lo[idx] = l;
}

// One thread per (row, head of [q | k | v], RoPE pair j < d/2).  The chunk
// partials and the RoPE table entries are loaded together, then summed in
// chunk order.
__global__ __launch_bounds__(256) void k_qkv_finish(const float* __restrict__ part, int kc, int M, int q_rows,
                                                    int Mp, int n_q, int n_kv, int d, const float* __restrict__ rc,
                                                    const float* __restrict__ rs, u16* __restrict__ q_hi,
                                                    u16* __restrict__ q_lo, u16* __restrict__ kv, int64_t kv_tiles,
                                                    SeqTable st) {
  const int half = d / 2, nh = n_q + 2 * n_kv, N = nh * d;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * nh * half) return;
  const int j = idx % half, t = idx / half;
  const int hh = t % nh, row = t / nh;
  if (hh < n_q && row >= q_rows) return;  // appended context rows: no q
  const int b = seq_of_row(st, row);
  const int pos = st.pos_base[b] + (row - st.row_start[b]);
  const bool rot = hh < n_q + n_kv;
  float cs = 1.f, sn = 0.f;
  if (rot) {
    cs = rc[(size_t)pos * half + j];
    sn = rs[(size_t)pos * half + j];
  }
  float pa[kMaxKc], pb[kMaxKc];
#pragma unroll
  for (int q = 0; q < kMaxKc; ++q)
    if (q < kc) {
      const float* p = part + ((size_t)q * Mp + row) * N + hh * d + j;
      pa[q] = p[0];
      pb[q] = p[half];
    }
  float a = 0.f, bv = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxKc; ++q)
    if (q < kc) {
      a += pa[q];
      bv += pb[q];
    }
  if (rot) {
    const float a2 = a * cs - bv * sn, b2 = bv * cs + a * sn;
    a = a2;
    bv = b2;
  }
  u16 ah, al, bh, bl;
  split_pair(a, ah, al);
  split_pair(bv, bh, bl);
  if (hh < n_q) {
    const size_t o = (size_t)row * (n_q * d) + hh * d + j;
    q_hi[o] = ah;
    q_lo[o] = al;
    q_hi[o + half] = bh;
    q_lo[o + half] = bl;
    return;
  }
  const int64_t slot = st.slot_base[b] + pos;
  if (hh < n_q + n_kv) {
    u16* p = kv_k_elem(kv, hh - n_q, slot, kv_tiles, d, j);
    p[0] = ah;
    p[kTileKeys * d] = al;
    p[half] = bh;
    p[kTileKeys * d + half] = bl;
  } else {
    u16* p = kv_v_elem(kv, hh - n_q - n_kv, slot, kv_tiles, d, j);
    u16* p2 = kv_v_elem(kv, hh - n_q - n_kv, slot, kv_tiles, d, j + half);
    p[0] = ah;
    p[kTileKeys * d] = al;
    p2[0] = bh;
    p2[kTileKeys * d] = bl;
  }
}

// Many-row form of k_qkv_finish: workgroup (64-row block, head) of the
// q|k|v heads.  q and K are written row by row; V goes through LDS so that
// each transposed V-plane row receives its slots from consecutive threads.
template <int D>
__global__ __launch_bounds__(256) void k_qkv_finish_blk(const float* __restrict__ part, int kc, int M, int Mp,
                                                        int n_q, int n_kv, const float* __restrict__ rc,
                                                        const float* __restrict__ rs, u16* __restrict__ q_hi,
                                                        u16* __restrict__ q_lo, u16* __restrict__ kv,
                                                        int64_t kv_tiles, SeqTable st) {
  constexpr int HALF = D / 2, R = 64, RSTEP = 256 / HALF;
  __shared__ u16 vh[D][R + 2], vl[D][R + 2];
  __shared__ int64_t slot_s[R];
  __shared__ int pos_s[R];
  const int tid = threadIdx.x;
  const int nh = n_q + 2 * n_kv, N = nh * D;
  const int nblk = (M + R - 1) / R;
  const int rb = blockIdx.x % nblk, hh = blockIdx.x / nblk;
  const int r0 = rb * R;
  const bool is_q = hh < n_q, is_k = !is_q && hh < n_q + n_kv;
  if (tid < R) {
    const int row = r0 + tid;
    if (row < M) {
      const int b = seq_of_row(st, row);
      const int pos = st.pos_base[b] + (row - st.row_start[b]);
      pos_s[tid] = pos;
      slot_s[tid] = st.slot_base[b] + pos;
    }
  }
  __syncthreads();
  const int j = tid % HALF;
  for (int rr = tid / HALF; rr < R && r0 + rr < M; rr += RSTEP) {
    const int row = r0 + rr;
    float a = 0.f, bv = 0.f;
    for (int q = 0; q < kc; ++q) {
      const float* p = part + ((size_t)q * Mp + row) * N + hh * D + j;
      a += p[0];
      bv += p[HALF];
    }
    if (!is_q && !is_k) {
      split_pair(a, vh[j][rr], vl[j][rr]);
      split_pair(bv, vh[j + HALF][rr], vl[j + HALF][rr]);
      continue;
    }
    const int pos = pos_s[rr];
    const float cs = rc[(size_t)pos * HALF + j], sn = rs[(size_t)pos * HALF + j];
    const float a2 = a * cs - bv * sn, b2 = bv * cs + a * sn;
    u16 ah, al, bh, bl;
    split_pair(a2, ah, al);
    split_pair(b2, bh, bl);
    if (is_q) {
      const size_t o = (size_t)row * (n_q * D) + hh * D + j;
      q_hi[o] = ah;
      q_lo[o] = al;
      q_hi[o + HALF] = bh;
      q_lo[o + HALF] = bl;
    } else {
      u16* p = kv_k_elem(kv, hh - n_q, slot_s[rr], kv_tiles, D, j);
      p[0] = ah;
      p[kTileKeys * D] = al;
      p[HALF] = bh;
      p[kTileKeys * D + HALF] = bl;
    }
  }
  if (is_q || is_k) return;  // uniform over the workgroup
  __syncthreads();
  const int rr = tid % R;
  if (r0 + rr < M) {
    const int64_t slot = slot_s[rr];
    for (int dd = tid / R; dd < D; dd += 256 / R) {
      u16* pv = kv_v_elem(kv, hh - n_q - n_kv, slot, kv_tiles, D, dd);
      pv[0] = vh[dd][rr];
      pv[kTileKeys * D] = vl[dd][rr];
    }
  }
}

// Workgroup (64-row block, layer, kv head): its rows' K pairs with RoPE and
// V values, summed over kc chunks in order.  K goes to the cache row by row
// (consecutive threads, consecutive dimensions); V, whose cache planes are
// transposed ([d][slot]), goes through LDS so that each V-plane row receives
// its 64 slots from consecutive threads.
template <int D>
__global__ __launch_bounds__(256) void k_kv_finish(const float* __restrict__ part, int kc, int M, int Mp,
                                                   int n_layers, int n_kv, const float* __restrict__ rc,
                                                   const float* __restrict__ rs, u16* __restrict__ kv0,
                                                   size_t layer_stride, int64_t kv_tiles, SeqTable st) {
  constexpr int HALF = D / 2, R = 64, RSTEP = 256 / HALF;
  __shared__ u16 vh[D][R + 2], vl[D][R + 2];
  __shared__ int64_t slot_s[R];
  __shared__ int pos_s[R];
  const int tid = threadIdx.x;
  const int nblk = (M + R - 1) / R;
  int t = blockIdx.x;
  const int rb = t % nblk;
  t /= nblk;
  const int gk = t % n_kv, l = t / n_kv;
  const int r0 = rb * R, kd = n_kv * D, N = n_layers * 2 * kd;
  u16* cache = kv0 + (size_t)l * layer_stride;
  if (tid < R) {
    const int row = r0 + tid;
    if (row < M) {
      const int b = seq_of_row(st, row);
      const int pos = st.pos_base[b] + (row - st.row_start[b]);
      pos_s[tid] = pos;
      slot_s[tid] = st.slot_base[b] + pos;
    }
  }
  __syncthreads();
  const int j = tid % HALF;
  for (int rr = tid / HALF; rr < R && r0 + rr < M; rr += RSTEP) {
    const int row = r0 + rr;
    float k1 = 0.f, k2 = 0.f, v1 = 0.f, v2 = 0.f;
    for (int q = 0; q < kc; ++q) {
      const float* p = part + ((size_t)q * Mp + row) * N + l * 2 * kd + gk * D + j;
      k1 += p[0];
      k2 += p[HALF];
      v1 += p[kd];
      v2 += p[kd + HALF];
    }
    const int pos = pos_s[rr];
    const float cs = rc[(size_t)pos * HALF + j], sn = rs[(size_t)pos * HALF + j];
    const float e1 = k1 * cs - k2 * sn, e2 = k2 * cs + k1 * sn;
    u16 h, lo;
    u16* pk = kv_k_elem(cache, gk, slot_s[rr], kv_tiles, D, j);
    split_pair(e1, h, lo);
    pk[0] = h;
    pk[kTileKeys * D] = lo;
    split_pair(e2, h, lo);
    pk[HALF] = h;
    pk[kTileKeys * D + HALF] = lo;
    split_pair(v1, vh[j][rr], vl[j][rr]);
    split_pair(v2, vh[j + HALF][rr], vl[j + HALF][rr]);
  }
  __syncthreads();
  const int rr = tid % R;
  if (r0 + rr < M) {
    const int64_t slot = slot_s[rr];
    for (int dd = tid / R; dd < D; dd += 256 / R) {
      u16* pv = kv_v_elem(cache, gk, slot, kv_tiles, D, dd);
      pv[0] = vh[dd][rr];
      pv[kTileKeys * D] = vl[dd][rr];
    }
  }
}

// draft[b][i-1] = lowest column of the largest logit of block row i: the
// largest of its n_parts partial keys (four independent loads per thread per
// step), then a wave and workgroup max.
__global__ __launch_bounds__(256) void k_argmax_reduce(const u64* __restrict__ part, int n_parts,
                                                       int Mp, int block, int32_t* __restrict__ draft) {
  const int dr = blockIdx.x;
  const int b = dr / (block - 1), i = dr % (block - 1) + 1;
  const int row = b * block + i;
  u64 best = 0;
  int t = threadIdx.x;
  for (; t + 768 < n_parts; t += 1024) {
    const u64 v0 = part[(size_t)t * Mp + row], v1 = part[(size_t)(t + 256) * Mp + row];
    const u64 v2 = part[(size_t)(t + 512) * Mp + row], v3 = part[(size_t)(t + 768) * Mp + row];
    const u64 m01 = v0 > v1 ? v0 : v1, m23 = v2 > v3 ? v2 : v3;
    const u64 m = m01 > m23 ? m01 : m23;
    best = m > best ? m : best;
  }
  for (; t < n_parts; t += 256) {
    const u64 v = part[(size_t)t * Mp + row];
    best = v > best ? v : best;
  }
  best = max_wave_u64(best);
  __shared__ u64 wbest[4];
  if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    u64 r = wbest[0];
    for (int w = 1; w < 4; ++w) r = wbest[w] > r ? wbest[w] : r;
    draft[dr] = (int32_t)(0xFFFFFFFFu - (uint32_t)(r & 0xFFFFFFFFull));
  }
}

// One wave per sequence: 64 positions are compared at once (all loads in
// flight together); the first chunk with a mismatch gives the accepted
// length, and the target token there (or at block - 1) the next anchor.
__global__ __launch_bounds__(256) void k_accept(const int32_t* __restrict__ draft,
                                                const int32_t* __restrict__ target, int n, int block,
                                                int32_t* __restrict__ accept,
                                                int32_t* __restrict__ next_anchor) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= n) return;
  const int32_t* dr = draft + (size_t)b * (block - 1);
  const int32_t* tg = target + (size_t)b * block;
  int k = -1, nxt = 0;
  for (int base = 0; base < block && k < 0; base += 64) {
    const int i = base + lane;
    const int t = i < block ? tg[i] : 0;
    const int d = i < block - 1 ? dr[i] : 0;
    const u64 miss = __ballot(i < block - 1 && d != t);
    int kk = -1;
    if (miss) kk = base + __builtin_ctzll(miss);
    else if (block - 1 < base + 64) kk = block - 1;
    if (kk >= 0) {
      k = kk;
      nxt = __shfl(t, kk - base, 64);
    }
  }
  if (lane == 0) {
    accept[b] = k;
    if (next_anchor) next_anchor[b] = nxt;
  }
}

// ---------------------------------------------------------------------------
// Lossless verification of sampled drafts (speculative sampling), fp64.
// The vocabulary is cut into C chunks.  k_verify_lse: workgroup (b, i, c)
// forms (max, sum of exp) of P_i / T and, for draft positions i < B, of
// Q_i / T over chunk c.  k_verify_keep: one workgroup per sequence, one
// wave per position, merges each position's chunk partials into its log
// normalisers,
// takes the keep test U q_i(x) < p_i(x) of the draft x and finds the first
// position k that fails (or the bonus position B).  k_verify_sample:
// workgroup (b, c) forms the largest log(max(0, p_k - q_k)) + G (or
// P_B / T + G) over its own, finer sampling chunk, lowest index on ties.
// k_verify_final: per sequence, the largest of the chunk candidates.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void amax_merge(double& v, int& ix, double v2, int ix2) {
  if (v2 > v || (v2 == v && ix2 < ix)) {
    v = v2;
    ix = ix2;
  }
}

int verify_chunks(int vocab) { return std::min(kVerifyMaxChunks, std::max(1, (vocab + 4095) / 4096)); }
int verify_rchunks(int vocab) { return std::min(kVerifyMaxRChunks, std::max(1, (vocab + 511) / 512)); }

// Chunk partial of the log normalisers: (max, sum) of P / T and of Q / T.
struct Lse4 {
  double mp, sp, mq, sq;
};

__device__ __forceinline__ double wave_max(double v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Workgroup (b, i, c): (max, sum of exp(x - max)) of x = P_i / T and, for
// i < B, Q_i / T over vocabulary chunk c.  A chunk holds at most 4096
// entries, so each thread loads its (at most 16) values of both rows at once
// into registers and both passes run there.
__global__ __launch_bounds__(256) void k_verify_lse(const float* __restrict__ ql, const float* __restrict__ pl,
                                                    int block, int vocab, int chunks, double inv_t,
                                                    Lse4* __restrict__ part) {
  constexpr int PER = 16;  // values per thread and row: 16 x 256 >= 4096
  __shared__ double sm[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x % chunks, bi = blockIdx.x / chunks;  // bi = b * block + (i - 1)
  const int b = bi / block, i = bi % block + 1;
  const bool has_q = i < block;
  const float* P = pl + (size_t)bi * vocab;
  const float* Q = has_q ? ql + ((size_t)b * (block - 1) + (i - 1)) * vocab : P;
  const int per = (vocab + chunks - 1) / chunks, v0 = c * per, v1 = min(vocab, v0 + per);
  float pv[PER], qv[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = v0 + tid + u * 256;
    pv[u] = v < v1 ? P[v] : -INFINITY;
    qv[u] = v < v1 ? Q[v] : -INFINITY;
  }
  float fp = -INFINITY, fq = -INFINITY;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    fp = fmaxf(fp, pv[u]);
    fq = fmaxf(fq, qv[u]);
  }
  double mp = wave_max((double)fp), mq = wave_max((double)fq);
  if (lane == 0) {
    sm[0][wave] = mp;
    sm[1][wave] = mq;
  }
  __syncthreads();
  mp = fmax(fmax(sm[0][0], sm[0][1]), fmax(sm[0][2], sm[0][3])) * inv_t;
  mq = fmax(fmax(sm[1][0], sm[1][1]), fmax(sm[1][2], sm[1][3])) * inv_t;
  __syncthreads();
  double sp = 0.0, sq = 0.0;
  if (v0 < v1) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (pv[u] != -INFINITY) sp += exp((double)pv[u] * inv_t - mp);
      if (qv[u] != -INFINITY) sq += exp((double)qv[u] * inv_t - mq);
    }
  }
  sp = wave_sum(sp);
  sq = wave_sum(sq);
  if (lane == 0) {
    sm[0][wave] = sp;
    sm[1][wave] = sq;
  }
  __syncthreads();
  if (tid == 0) {
    sp = (sm[0][0] + sm[0][1]) + (sm[0][2] + sm[0][3]);
    sq = (sm[1][0] + sm[1][1]) + (sm[1][2] + sm[1][3]);
    part[(size_t)bi * chunks + c] = has_q ? Lse4{mp, sp, mq, sq} : Lse4{mp, sp, -INFINITY, 0.0};
  }
}

// Log normalisers (log Z_p, log Z_q) of position bi from its chunk
// partials, by one wave: lane c holds chunk c (chunks <= 64); the largest
// chunk maximum first, then one exp per chunk, summed by a fixed shuffle tree.
__device__ __forceinline__ void verify_lz_wave(const Lse4* part, int bi, int chunks, int lane, double& lzp,
                                               double& lzq) {
  Lse4 t{-INFINITY, 0.0, -INFINITY, 0.0};
  if (lane < chunks) t = part[(size_t)bi * chunks + lane];
  const double mp = wave_max(t.mp), mq = wave_max(t.mq);
  const double sp = wave_sum(t.mp == -INFINITY ? 0.0 : t.sp * exp(t.mp - mp));
  const double sq = wave_sum(t.mq == -INFINITY ? 0.0 : t.sq * exp(t.mq - mq));
  lzp = mp + log(sp);
  lzq = mq + log(sq);
}

// Per verification record (per sequence): the first rejected position k
// (block when every draft is kept) and the log normalisers at k.
struct VerifyPos {
  double lzp, lzq;
  int k, pad;
};

// One workgroup of 16 waves per sequence: wave w handles draft positions
// i = w + 1, w + 17, ...: its log normalisers and the keep test
// U q_i(x) < p_i(x); then thread 0 takes the first failing position.
__global__ __launch_bounds__(1024) void k_verify_keep(const int32_t* __restrict__ draft, const float* __restrict__ ql,
                                                      const float* __restrict__ pl, int block, int vocab, int chunks,
                                                      double inv_t, u64 seed, const Lse4* __restrict__ part,
                                                      VerifyPos* __restrict__ vp, int32_t* __restrict__ accept) {
  __shared__ int keep[1024];
  __shared__ double lz[1024][2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, b = blockIdx.x;
  for (int i = 1 + wave; i < block; i += 16) {
    const int bi = b * block + (i - 1);
    int x = 0;
    if (lane == 0) x = min(max(draft[(size_t)b * (block - 1) + (i - 1)], 0), vocab - 1);
    double lzp, lzq;
    verify_lz_wave(part, bi, chunks, lane, lzp, lzq);
    if (lane == 0) {
      const double px = exp((double)pl[(size_t)bi * vocab + x] * inv_t - lzp);
      const double qx = exp((double)ql[((size_t)b * (block - 1) + (i - 1)) * vocab + x] * inv_t - lzq);
      keep[i] = philox_uniform(seed, kPurposeAccept, b, i, 0) * qx < px;
      lz[i][0] = lzp;
      lz[i][1] = lzq;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int k = 1;
    while (k < block && keep[k]) ++k;  // first rejected position, or block (bonus)
    VerifyPos r;
    r.k = k;
    r.pad = 0;
    r.lzp = k < block ? lz[k][0] : 0.0;
    r.lzq = k < block ? lz[k][1] : 0.0;
    vp[b] = r;
    accept[b] = k - 1;
  }
}

// Workgroup (b, c): chunk c's largest log(max(0, p_k - q_k)) + G at the
// first rejected position k, or P_B / T + G at the bonus position.
__global__ __launch_bounds__(256) void k_verify_sample(const float* __restrict__ ql, const float* __restrict__ pl,
                                                       int block, int vocab, int rchunks, double inv_t, u64 seed,
                                                       const VerifyPos* __restrict__ vp,
                                                       double* __restrict__ cand_v, int* __restrict__ cand_i) {
  __shared__ double sv[4];
  __shared__ int si[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x % rchunks, b = blockIdx.x / rchunks;
  const VerifyPos r = vp[b];
  const int k = r.k;
  const bool bonus = k == block;
  const float* P = pl + ((size_t)b * block + (k - 1)) * vocab;
  const float* Q = bonus ? nullptr : ql + ((size_t)b * (block - 1) + (k - 1)) * vocab;
  const int per = (vocab + rchunks - 1) / rchunks, v0 = c * per, v1 = min(vocab, v0 + per);
  double best = -INFINITY;
  int bix = vocab;
  for (int v = v0 + tid; v < v1; v += 256) {
    double sc;
    if (bonus) {
      sc = (double)P[v] * inv_t;
    } else {
      const double d = exp((double)P[v] * inv_t - r.lzp) - exp((double)Q[v] * inv_t - r.lzq);
      sc = d > 0.0 ? log(d) : -INFINITY;
    }
    if (sc == -INFINITY) continue;
    sc += gumbel(philox_uniform(seed, kPurposeResidual, b, k, v));
    amax_merge(best, bix, sc, v);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    const double ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bix, o, 64);
    amax_merge(best, bix, ov, oi);
  }
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bix;
  }
  __syncthreads();
  if (tid == 0) {
    best = sv[0];
    bix = si[0];
    for (int w = 1; w < 4; ++w) amax_merge(best, bix, sv[w], si[w]);
    cand_v[(size_t)b * rchunks + c] = best;
    cand_i[(size_t)b * rchunks + c] = bix;
  }
}

// One wave per sequence: the largest chunk candidate (lowest index on ties).
__global__ __launch_bounds__(256) void k_verify_final(const double* __restrict__ cand_v,
                                                      const int* __restrict__ cand_i, int n, int chunks,
                                                      int vocab, int32_t* __restrict__ next_token) {
  const int lane = threadIdx.x & 63, b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= n) return;
  double best = -INFINITY;
  int bix = vocab;
  for (int c = lane; c < chunks; c += 64) amax_merge(best, bix, cand_v[(size_t)b * chunks + c], cand_i[(size_t)b * chunks + c]);
  for (int o = 32; o >= 1; o >>= 1) {
    const double ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bix, o, 64);
    amax_merge(best, bix, ov, oi);
  }
  if (lane == 0) next_token[b] = bix < vocab ? bix : 0;
}


// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_resid_norm(float* x, const float* part, int kc, int part_rows, const int32_t* anchors,
                             const int32_t* block_tokens, const u16* embed, int block, int mask_id, int vocab,
                             const u16* gain, u16* out_hi, u16* out_lo, int H, int M, int out_rows, float eps,
                             hipStream_t s) {
  if (kc > kMaxKc || out_rows < M || H % 4 || H > kMaxHidden) return hipErrorInvalidValue;
  if (out_rows == 0) return hipSuccess;
  const dim3 grid(out_rows), blk(1024);
  if (H <= 4096)
    hipLaunchKernelGGL(k_resid_norm<1>, grid, blk, 0, s, x, part, kc, part_rows, anchors, block_tokens, embed, block,
                       mask_id, vocab, gain, out_hi, out_lo, H, M, eps);
  else if (H <= 8192)
    hipLaunchKernelGGL(k_resid_norm<2>, grid, blk, 0, s, x, part, kc, part_rows, anchors, block_tokens, embed, block,
                       mask_id, vocab, gain, out_hi, out_lo, H, M, eps);
  else
    hipLaunchKernelGGL(k_resid_norm<4>, grid, blk, 0, s, x, part, kc, part_rows, anchors, block_tokens, embed, block,
                       mask_id, vocab, gain, out_hi, out_lo, H, M, eps);
  return hipGetLastError();
}

// SwiGLU over the K-chunk partial sums of the interleaved gate|up tiles
// (16-column tile t holds gate rows 8t..8t+7, then up rows 8t..8t+7): thread
// i takes outputs 4i..4i+3 of a row, sums each chunk's gate and up in chunk
// order and writes silu(g) u as hi/lo planes [row][ldh]; rows >= M are zero.
__global__ __launch_bounds__(256) void k_swiglu_finish(const float* __restrict__ part, int kc, int Mp, int M, int I,
                                                       u16* __restrict__ out_hi, u16* __restrict__ out_lo, int ldh) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x, per = (size_t)I / 4;
  if (idx >= (size_t)Mp * per) return;
  const int row = (int)(idx / per), j = (int)(idx % per) * 4;
  uint2 hw = make_uint2(0u, 0u), lw = make_uint2(0u, 0u);
  if (row < M) {
    const size_t col = (size_t)(j >> 3) * 16 + (j & 7), N = (size_t)2 * I;
    f32x4 ga[kMaxKc], ua[kMaxKc];
#pragma unroll
    for (int q = 0; q < kMaxKc; ++q)
      if (q < kc) {
        const float* p = part + ((size_t)q * Mp + row) * N + col;
        ga[q] = *reinterpret_cast<const f32x4*>(p);
        ua[q] = *reinterpret_cast<const f32x4*>(p + 8);
      }
    f32x4 gt = f32x4{0.f, 0.f, 0.f, 0.f}, up = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kMaxKc; ++q)
      if (q < kc) {
        gt += ga[q];
        up += ua[q];
      }
    u16 h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_pair(gt[i] / (1.0f + expf(-gt[i])) * up[i], h[i], l[i]);
    hw = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
    lw = make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
  }
  *reinterpret_cast<uint2*>(out_hi + (size_t)row * ldh + j) = hw;
  *reinterpret_cast<uint2*>(out_lo + (size_t)row * ldh + j) = lw;
}

// K chunks of a many-row SwiGLU projection: two when its 256 x 192 tiles
// split in two still fill at most one round of one workgroup per CU (256
// rows at I = 12288: 128 tiles, 256 workgroups); unsplit such a shape runs
// 128 x 192 tiles.  The two chunks' partials then meet in k_swiglu_finish
// (block-32 batch of eight sequences, per layer: 119.5 us unsplit against
// 98.1 + 12.5 us, draft pass 1.502 -> 1.490 ms, same box).
int swiglu_kc(int n_tiles, int K, int Mp) {
  if (Mp <= 32 || Mp % 256 || K % 64 || n_tiles % 12) return 1;
  return (Mp / 256) * (n_tiles / 12) * 2 <= 256 ? 2 : 1;
}

hipError_t launch_reduce_split(const float* part, int kc, int part_rows, int N, u16* out_hi, u16* out_lo, int M,
                               int out_rows, hipStream_t s) {
  const size_t total = (size_t)out_rows * N;
  hipLaunchKernelGGL(k_reduce_split, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, kc, part_rows, N,
                     out_hi, out_lo, M, out_rows);
  return hipGetLastError();
}

hipError_t launch_qkv_finish(const float* part, int kc, int M, int q_rows, int Mp, int n_q, int n_kv, int head_dim,
                             const float* rope_cos, const float* rope_sin, u16* q_hi, u16* q_lo,
                             u16* kv_cache, int64_t kv_tiles, const SeqTable& st, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (M >= 1024 && (head_dim == 128 || head_dim == 64)) {  // many rows: 64-row blocks per head
    // this form finishes q for every row; rows without q partials (q_rows <
    // M, appended rows of a fused few-row step) never reach it
    if (q_rows < M) return hipErrorInvalidValue;
    const dim3 grid((M + 63) / 64 * (n_q + 2 * n_kv));
    if (head_dim == 128)
      hipLaunchKernelGGL(k_qkv_finish_blk<128>, grid, dim3(256), 0, s, part, kc, M, Mp, n_q, n_kv, rope_cos,
                         rope_sin, q_hi, q_lo, kv_cache, kv_tiles, st);
    else
      hipLaunchKernelGGL(k_qkv_finish_blk<64>, grid, dim3(256), 0, s, part, kc, M, Mp, n_q, n_kv, rope_cos,
                         rope_sin, q_hi, q_lo, kv_cache, kv_tiles, st);
    return hipGetLastError();
  }
  if (kc > kMaxKc) return hipErrorInvalidValue;
  const int total = M * (n_q + 2 * n_kv) * (head_dim / 2);
  hipLaunchKernelGGL(k_qkv_finish, dim3((total + 255) / 256), dim3(256), 0, s, part, kc, M, q_rows, Mp, n_q, n_kv,
                     head_dim, rope_cos, rope_sin, q_hi, q_lo, kv_cache, kv_tiles, st);
  return hipGetLastError();
}

hipError_t launch_kv_finish(const float* part, int kc, int M, int Mp, int n_layers, int n_kv, int head_dim,
                            const float* rope_cos, const float* rope_sin, u16* kv_cache0, size_t layer_stride,
                            int64_t kv_tiles, const SeqTable& st, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const dim3 grid((M + 63) / 64 * n_layers * n_kv);
  if (head_dim == 128)
    hipLaunchKernelGGL(k_kv_finish<128>, grid, dim3(256), 0, s, part, kc, M, Mp, n_layers, n_kv, rope_cos, rope_sin,
                       kv_cache0, layer_stride, kv_tiles, st);
  else if (head_dim == 64)
    hipLaunchKernelGGL(k_kv_finish<64>, grid, dim3(256), 0, s, part, kc, M, Mp, n_layers, n_kv, rope_cos, rope_sin,
                       kv_cache0, layer_stride, kv_tiles, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

GemmPlan gemm_plan(int n_tiles, int K, int Mp, bool may_split) {
  GemmPlan p;
  p.kc = 1;
  if (Mp <= 32) {
    p.nc = (n_tiles % 8 == 0 && n_tiles >= 1024) ? 8 : (n_tiles % 4 == 0 ? 4 : (n_tiles % 2 == 0 ? 2 : 1));
    p.ks = kSkinnyWaves;
    // wide unsplit outputs: six column tiles when that, and not eight, gives
    // whole waves of workgroups over the 256 CUs (SwiGLU at I = 12288: 256
    // workgroups instead of 192, 39.9 -> 38.6 us with cold weights)
    if (!may_split && n_tiles >= 1024 && n_tiles % 6 == 0 && (n_tiles / 6) % 256 == 0 && (n_tiles / 8) % 256 != 0)
      p.nc = 6;
    if (may_split) {
      // narrow split-K outputs (O, down, fusion at H = 4096): eight column
      // tiles and eight waves per workgroup stream a little faster (down
      // projection 25.0 -> 22.8 us, fusion 38.0 -> 35.0 us, cold weights)
      if (n_tiles % 8 == 0 && n_tiles <= 256 && K % (8 * 8 * 64) == 0) {
        p.nc = 8;
        p.ks = 8;
      }
      const int waves = n_tiles / p.nc * p.ks;
      const int chunk = p.ks * 64;  // K granularity of one chunk: 64 per wave
      while (p.kc * 2 <= kMaxKc && p.kc * 2 * waves <= 3072 && K % (p.kc * 2 * chunk) == 0) p.kc *= 2;
    }
  } else {
    p.ks = 0;
    p.nc = kBigBN / 16;
    // K chunks for about 256 workgroups of 128-row tiles (128 of 256-row
    // tiles): fewer partial sums to write and re-read than with 512 (draft
    // pass of eight ragged block-32 sequences 1.647 -> 1.582 ms, of 32
    // sequences 3.767 -> 3.716-3.748 ms).  Long K ranges, where the partial
    // sums weigh little against the products, keep about 512 (the fusion
    // map, K 20480, at 1024 rows: 256 workgroups made the ingest of 1024
    // positions 0.39 -> 0.48 ms)
    if (may_split) {
      const int wgs = (Mp / 128) * ((n_tiles + p.nc - 1) / p.nc), cap = K >= 16384 ? 512 : 256;
      while (p.kc * 2 <= kMaxKc && p.kc * 2 * wgs <= cap && K % (p.kc * 2 * 32) == 0) p.kc *= 2;
    }
  }
  return p;
}

template <int EPI, int MAP, bool SPLIT, int RG, bool PK>
static hipError_t skinny_nc(const GemmArgs& g, const SeqTable& st, const GemmPlan& p, hipStream_t s) {
  const dim3 grid(g.n_tiles / p.nc, p.kc), blk(p.ks * 64);
  if constexpr (MAP == MAP_QKV && RG == 2 && EPI == EPI_PARTIAL) {
    const int qt = g.ep.n_q * g.ep.head_dim / 16;  // q column tiles, a whole number of groups
    if (g.q_rows > 0 && g.q_rows <= 16 && p.ks == kSkinnyWaves && p.nc == 4 && qt % 4 == 0 && qt < g.n_tiles) {
      hipLaunchKernelGGL((k_skinny_qkv_rows<4, SPLIT, kSkinnyWaves, PK>), grid, blk, 0, s, g, st, qt / 4);
      return hipGetLastError();
    }
  }
  if (p.ks == 8) {
    if (p.nc == 8) {
      hipLaunchKernelGGL((k_skinny<EPI, MAP, 8, RG, SPLIT, 8, PK>), grid, blk, 0, s, g, st);
      return hipGetLastError();
    }
    if constexpr (EPI == EPI_SWIGLU) {
      if (p.nc == 6) {
        hipLaunchKernelGGL((k_skinny<EPI, MAP, 6, RG, SPLIT, 8, PK>), grid, blk, 0, s, g, st);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  }
  if (p.ks != kSkinnyWaves) return hipErrorInvalidValue;
  switch (p.nc) {
    case 8: hipLaunchKernelGGL((k_skinny<EPI, MAP, 8, RG, SPLIT, kSkinnyWaves, PK>), grid, blk, 0, s, g, st); break;
    case 4: hipLaunchKernelGGL((k_skinny<EPI, MAP, 4, RG, SPLIT, kSkinnyWaves, PK>), grid, blk, 0, s, g, st); break;
    case 2: hipLaunchKernelGGL((k_skinny<EPI, MAP, 2, RG, SPLIT, kSkinnyWaves, PK>), grid, blk, 0, s, g, st); break;
    default: hipLaunchKernelGGL((k_skinny<EPI, MAP, 1, RG, SPLIT, kSkinnyWaves, PK>), grid, blk, 0, s, g, st); break;
  }
  return hipGetLastError();
}

// Column tiles [nt0, nt0 + nt) of width BN (nt < 0: all from nt0 on); an
// argmax epilogue stores tile nt0 + i's partial keys in slot slot0 + i
// (slot0 < 0: slot nt0 + i).
template <int EPI, int MAP, bool SPLIT, int BM, int WM, int WN, int S, int BN = kBigBN>
static hipError_t dl_launch(const GemmArgs& g, const SeqTable& st, int Mp, const GemmPlan& p, hipStream_t s,
                            int nt0 = 0, int nt = -1, int slot0 = -1) {
  if (Mp % BM || g.K % (p.kc * 32) || g.a_rows < 1) return hipErrorInvalidValue;
  const int mt = Mp / BM, nt_all = (g.n_tiles + BN / 16 - 1) / (BN / 16);
  if (nt < 0) nt = nt_all - nt0;
  if (nt0 < 0 || nt < 1 || nt0 + nt > nt_all) return hipErrorInvalidValue;
  const int wgs = mt * p.kc * nt, padded = (wgs + 7) / 8 * 8;
  hipLaunchKernelGGL((k_gemm_dl<EPI, MAP, SPLIT, BM, WM, WN, S, BN>), dim3(padded), dim3(WM * WN * 64), 0, s, g,
                     st, mt, p.kc, nt0, nt0 + nt, slot0 < 0 ? nt0 : slot0);
  return hipGetLastError();
}

// Tile shape per launch: 256-row tiles (sixteen waves of 64 x 64, three
// stages, one workgroup per CU) when the rows allow and the grid still
// covers the CUs; else 128-row tiles (eight waves of 64 x 64) with two
// stages of at most 32 KB, so that two workgroups share a CU, when the grid
// covers the CUs, and with four stages (one per CU) on a smaller grid, which
// the dispatcher would otherwise pack two to a CU, leaving CUs idle (at 192
// workgroups: 162 us with two stages, 138 us with four).
// Column width of the many-row LM head's 256-row tiles: 240 (twelve waves of
// 64 x 80 columns) when its whole rounds over the CUs take less time than
// 256's (round times 201 and 210 us at K 4096); the argmax partials are
// counted per tile of this width.  151,936 columns at 256 rows: 634 tiles
// (2.48 rounds) instead of 594 (2.32), 643.6 -> 607.4 us; at 512 rows 1068
// -> 1034 us; the per-row keys are the same.
static int lm_head_bn(int n_tiles, int Mp) {
  const long mt = Mp / 256, t256 = (n_tiles + 15) / 16, t240 = (n_tiles + 14) / 15;
  if (Mp % 256 || mt * t256 < 256) return kBigBN;  // not a 256-row-tile launch
  return (mt * t240 + 255) / 256 * 201 < (mt * t256 + 255) / 256 * 210 ? 240 : kBigBN;
}

// A last round of 240-column tiles that is at most half full: the columns
// past the whole rounds (*nm tiles of 240) go to a second launch of 128 x 256
// tiles with four stages (eight waves of 64 x 64, one workgroup per CU), one
// round of which takes about two thirds of a round of 256 x 240 tiles.  It
// needs the split on a 256-column boundary.  Returns the second launch's
// column tiles (0: one launch).
static int lm_head_tail(int n_tiles, int Mp, int* nm) {
  *nm = 0;
  if (lm_head_bn(n_tiles, Mp) != 240) return 0;
  const int mt = Mp / 256, t240 = (n_tiles + 14) / 15, wgs = mt * t240, full = wgs / 256 * 256;
  if (full == wgs || full % mt) return 0;
  const int main_tiles = full / mt;
  if (main_tiles % 16) return 0;  // 240 * main_tiles not a multiple of 256
  const int tail = (n_tiles - main_tiles * 15 + 15) / 16;
  if (2 * mt * tail > 256) return 0;
  *nm = main_tiles;
  return tail;
}

template <int EPI, int MAP, bool SPLIT>
static hipError_t dl_dispatch(const GemmArgs& g, const SeqTable& st, int Mp, const GemmPlan& p, hipStream_t s) {
  if constexpr (SPLIT && EPI != EPI_ARGMAX && EPI != EPI_SAMPLE) {
    // hi/lo activations: the tile shape whose whole rounds of workgroups
    // over the CUs take least time.  A round's time per shape (us at K 4096,
    // SwiGLU projection, one box): 256 x 256 three stages 210, 256 x 192
    // 177, 128-row tiles with two stages (two workgroups per CU) 236 (x 256)
    // and 195 (x 192), with four stages (one per CU) 130 and 119.  So 512
    // rows of the SwiGLU projection take one round of 256 x 192 tiles
    // (214.8 -> 177.5 us), 256 rows one of 128 x 192 (130.0 -> 119.3 us).
    // The K chunks stay the plan's, which sized the partial buffers; the
    // column tiles of any width sum their K range in the same order, so
    // every shape gives the same bits.  The argmax epilogues take their
    // width from lm_head_bn and lm_head_tail, which argmax_parts also uses
    // to count their per-workgroup partials.
    struct Shape { int bm, bn, per_cu, round_us; };
    const Shape shapes[6] = {{256, 256, 1, 210}, {256, 192, 1, 177}, {128, 256, 2, 236},
                             {128, 192, 2, 195}, {128, 256, 1, 130}, {128, 192, 1, 119}};
    int best = -1;
    long best_t = 0;
    for (int i = 0; i < 6; ++i) {
      if (Mp % shapes[i].bm) continue;
      const long wgs = (long)(Mp / shapes[i].bm) * p.kc * ((g.n_tiles + shapes[i].bn / 16 - 1) / (shapes[i].bn / 16));
      const long t = (wgs + 256 * shapes[i].per_cu - 1) / (256 * shapes[i].per_cu) * shapes[i].round_us;
      if (best < 0 || t < best_t) best = i, best_t = t;
    }
    switch (best) {
      case 0: return dl_launch<EPI, MAP, SPLIT, 256, 4, 4, 3>(g, st, Mp, p, s);
      case 1: return dl_launch<EPI, MAP, SPLIT, 256, 4, 4, 3, 192>(g, st, Mp, p, s);
      case 2: return dl_launch<EPI, MAP, SPLIT, 128, 2, 4, 2>(g, st, Mp, p, s);
      case 3: return dl_launch<EPI, MAP, SPLIT, 128, 2, 4, 2, 192>(g, st, Mp, p, s);
      case 4: return dl_launch<EPI, MAP, SPLIT, 128, 2, 4, 4>(g, st, Mp, p, s);
      case 5: return dl_launch<EPI, MAP, SPLIT, 128, 2, 4, 4, 192>(g, st, Mp, p, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int nt = (g.n_tiles + p.nc - 1) / p.nc;
  if (Mp % 256 == 0 && (Mp / 256) * nt * p.kc >= 256) {
    if constexpr (EPI == EPI_ARGMAX || EPI == EPI_SAMPLE)
      if (lm_head_bn(g.n_tiles, Mp) == 240) {
        int nm;
        if (const int tail = lm_head_tail(g.n_tiles, Mp, &nm)) {
          // partial keys: slots 0 .. nm-1 for the 240-column tiles, then
          // one per 256-column tile of the tail
          const hipError_t e = dl_launch<EPI, MAP, SPLIT, 256, 4, 3, 3, 240>(g, st, Mp, p, s, 0, nm);
          if (e != hipSuccess) return e;
          return dl_launch<EPI, MAP, SPLIT, 128, 2, 4, 4>(g, st, Mp, p, s, nm * 15 / 16, tail, nm);
        }
        return dl_launch<EPI, MAP, SPLIT, 256, 4, 3, 3, 240>(g, st, Mp, p, s);
      }
    return dl_launch<EPI, MAP, SPLIT, 256, 4, 4, 3>(g, st, Mp, p, s);
  }
  if ((Mp / 128) * nt * p.kc >= 256) return dl_launch<EPI, MAP, SPLIT, 128, 2, 4, 2>(g, st, Mp, p, s);
  return dl_launch<EPI, MAP, SPLIT, 128, 2, 4, 4>(g, st, Mp, p, s);
}

template <int EPI, int MAP, bool SPLIT>
static hipError_t gemm_dispatch(const GemmArgs& g, const SeqTable& st, int Mp, hipStream_t s) {
  GemmPlan p = gemm_plan(g.n_tiles, g.K, Mp, EPI == EPI_PARTIAL);
  // the SwiGLU projection keeps more loads in flight with eight waves per
  // workgroup: 44.8 -> 40.5 us over packed weights (cold, 192 workgroups at
  // I = 12288), unchanged over row-major ones.  The LM head stays at four
  // (eight: 218.9 instead of 216.3 us in the decode step)
  if (EPI == EPI_SWIGLU && Mp <= 32 && (p.nc == 8 || p.nc == 6) && g.K % (8 * 64) == 0) p.ks = 8;
  if (Mp <= 32) {
    if (g.K % (p.kc * p.ks * 64) || Mp % 16) return hipErrorInvalidValue;
    if (g.wpack) {
      if (MAP == MAP_KVL) return hipErrorInvalidValue;  // never packed
      return Mp <= 16 ? skinny_nc<EPI, MAP, SPLIT, 1, true>(g, st, p, s)
                      : skinny_nc<EPI, MAP, SPLIT, 2, true>(g, st, p, s);
    }
    return Mp <= 16 ? skinny_nc<EPI, MAP, SPLIT, 1, false>(g, st, p, s)
                    : skinny_nc<EPI, MAP, SPLIT, 2, false>(g, st, p, s);
  }
  if (Mp % 128) return hipErrorInvalidValue;
  return dl_dispatch<EPI, MAP, SPLIT>(g, st, Mp, p, s);
}

hipError_t launch_gemm(const GemmArgs& g, const SeqTable& st, int Mp, hipStream_t s) {
  const bool split = g.a_lo != nullptr;
  // the norm factor of a SwiGLU launch (16 rows only) is read with one
  // 16-byte load per lane
  if (g.epi == EPI_SWIGLU && g.ep.ssq_in && (Mp > 16 || g.ep.n_ssq > 256 || g.ep.n_ssq % 4 || g.ep.norm_n < 1))
    return hipErrorInvalidValue;
  switch (g.epi) {
    case EPI_RESID:
      if (!gemm_whole_k_fits(g.n_tiles, g.K, Mp) || g.map != MAP_PLAIN || !split || (g.wpack && g.pk_kmajor))
        return hipErrorInvalidValue;
      return g.wpack ? whole_k_launch<true>(g, s) : whole_k_launch<false>(g, s);
    case EPI_SWIGLU:
      if (split && g.ep.out_f32 && swiglu_kc(g.n_tiles, g.K, Mp) == 2) {
        // two K chunks of partial sums into out_f32 ([2][Mp][16 n_tiles]),
        // then SwiGLU over them
        if (g.ep.ldh != g.n_tiles * 8 || g.ep.ldh % 4 || g.ep.ssq_in) return hipErrorInvalidValue;
        GemmArgs gp = g;
        gp.epi = EPI_PARTIAL;
        gp.ep.ldo = g.n_tiles * 16;
        GemmPlan p;
        p.kc = 2;
        p.nc = 12;
        p.ks = 0;
        const hipError_t e = dl_launch<EPI_PARTIAL, MAP_SWIGLU, true, 256, 4, 4, 3, 192>(gp, st, Mp, p, s);
        if (e != hipSuccess) return e;
        const size_t total = (size_t)Mp * (g.ep.ldh / 4);
        hipLaunchKernelGGL(k_swiglu_finish, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, g.ep.out_f32, 2,
                           Mp, g.ep.M, g.ep.ldh, g.ep.out_hi, g.ep.out_lo, g.ep.ldh);
        return hipGetLastError();
      }
      return gemm_dispatch<EPI_SWIGLU, MAP_SWIGLU, true>(g, st, Mp, s);
    case EPI_ARGMAX:  // greedy drafts, or sampled ones (the Gumbel code only where it runs)
      return g.ep.temp > 0.0 ? gemm_dispatch<EPI_SAMPLE, MAP_PLAIN, true>(g, st, Mp, s)
                             : gemm_dispatch<EPI_ARGMAX, MAP_PLAIN, true>(g, st, Mp, s);
    case EPI_PARTIAL:
      if (g.map == MAP_QKV) return gemm_dispatch<EPI_PARTIAL, MAP_QKV, true>(g, st, Mp, s);
      if (g.map == MAP_KVL) return gemm_dispatch<EPI_PARTIAL, MAP_KVL, true>(g, st, Mp, s);
      return split ? gemm_dispatch<EPI_PARTIAL, MAP_PLAIN, true>(g, st, Mp, s)
                   : gemm_dispatch<EPI_PARTIAL, MAP_PLAIN, false>(g, st, Mp, s);
    default:
      return hipErrorInvalidValue;
  }
}

// Workspace bound on the key splits of one call over `pairs` (sequence or
// group of blocks, kv head) pairs: about 512 workgroups.
int attention_max_splits(int pairs) {
  const int s = (512 + pairs - 1) / pairs;
  return s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
}

// Key splits of one call (at most max_splits), evened out so that no split of
// the longest unit (max_tiles tiles) is left empty.  One-block units: each
// split of the longest unit takes about unit_tiles / 192 tiles, the call's
// whole tile work (unit_tiles: tiles summed over units and kv heads) spread
// over three quarters of the CUs; that keeps ragged batches from waiting on
// their longest sequence (block 32, eight contexts of 512..4096: 7 splits,
// 1.4% faster per step than 4).  Grouped units (workgroups of up to sixteen
// waves): about 256 workgroups over the pairs.  Longer splits beat more of
// them once the work fills the chip: 8192 keys, 26 splits of five tiles 23.7
// us per layer against 43 of three 25.1 us, and 22 of six (the 192 rule)
// against 26 of five, draft pass 0.733 -> 0.726 ms; 32 of four, 20.1 against
// 18.2 us per layer; the training forward 1% faster per step with one split
// than with two.  Every unit's splits are its own tiles evened out over the
// split count: splits sized to the longest unit's share for every unit (a
// shorter unit leaving its later splits empty) measured slower on the
// ragged block-32 batch (1.600 against 1.663 ms at the same split count).
int attention_splits(int pairs, int max_tiles, int64_t unit_tiles, bool grouped, int max_splits) {
  if (max_tiles < 1) return 1;
  int s;
  if (grouped) {
    s = (256 + pairs - 1) / pairs;
  } else {
    const int64_t tps = std::max<int64_t>(1, (unit_tiles + 191) / 192);
    s = (int)((max_tiles + tps - 1) / tps);
  }
  s = std::max(1, std::min({s, max_splits, kMaxSplits, max_tiles}));
  const int tps = (max_tiles + s - 1) / s;
  return (max_tiles + tps - 1) / tps;
}

size_t attention_partial_bytes(int n_seqs, int n_q, int qtiles, int splits, int head_dim) {
  return (size_t)n_seqs * n_q * qtiles * splits * 16 * head_dim * sizeof(float);
}

size_t attention_ml_bytes(int n_seqs, int n_q, int qtiles, int splits) {
  return (size_t)n_seqs * n_q * qtiles * splits * 32 * sizeof(float);
}

template <int D, bool GRP, int HPW, bool HV, typename GT>
static hipError_t attention_tiles(int nw, dim3 grid, const u16* q_hi, const u16* q_lo, const u16* kv,
                                  int64_t kv_tiles, const u16* bkv, int bkv_tiles, float* part_o, float* part_ml,
                                  u16* o_hi, u16* o_lo, int block, int n_q, int n_kv, int splits, float scale,
                                  const SeqTable& st, const GT& grp, hipStream_t s) {
  if (nw <= 4)
    hipLaunchKernelGGL((k_attn_tiles<D, 4, GRP, HPW, HV>), grid, dim3(256), 0, s, q_hi, q_lo, kv, kv_tiles, bkv,
                       bkv_tiles, part_o, part_ml, o_hi, o_lo, block, n_q, n_kv, splits, scale, st, grp);
  else if (nw <= 8)
    hipLaunchKernelGGL((k_attn_tiles<D, 8, GRP, HPW, HV>), grid, dim3(512), 0, s, q_hi, q_lo, kv, kv_tiles, bkv,
                       bkv_tiles, part_o, part_ml, o_hi, o_lo, block, n_q, n_kv, splits, scale, st, grp);
  else if (nw <= 16)
    hipLaunchKernelGGL((k_attn_tiles<D, 16, GRP, HPW, HV>), grid, dim3(1024), 0, s, q_hi, q_lo, kv, kv_tiles, bkv,
                       bkv_tiles, part_o, part_ml, o_hi, o_lo, block, n_q, n_kv, splits, scale, st, grp);
  else
    return hipErrorInvalidValue;
  return hipSuccess;
}

template <int D>
static hipError_t attention_dispatch(const u16* q_hi, const u16* q_lo, const u16* kv, int64_t kv_tiles,
                                     const u16* bkv, float* part_o, float* part_ml, u16* o_hi, u16* o_lo, int n_seqs,
                                     int block, int n_q, int n_kv, int splits, int max_tiles, const SeqTable& st,
                                     const AttnGroups* groups, hipStream_t s) {
  const float scale = (float)(1.0 / sqrt((double)D));
  const int hpw = attention_heads_per_wave(n_q, n_kv, groups != nullptr);
  const int upb = (n_q / n_kv / hpw) * ((block + 15) / 16);  // query waves per block
  hipError_t e;
  if (groups) {
    const int nw = attention_group_size(n_q, n_kv, block) * upb;
    const dim3 grid(n_kv * splits, groups->n);
#define DFLASH_ATTN_GRP(H)                                                                                         \
  attention_tiles<D, true, H, false>(nw, grid, q_hi, q_lo, kv, kv_tiles, bkv, n_seqs, part_o, part_ml, o_hi, o_lo, block, \
                              n_q, n_kv, splits, scale, st, *groups, s)
    e = hpw == 2 ? DFLASH_ATTN_GRP(2) : DFLASH_ATTN_GRP(1);
#undef DFLASH_ATTN_GRP
  } else {
    // two waves per query unit, each taking half of every tile's keys, when
    // splits hold several tiles (32 sequences: 133.0 -> 122.3 us per layer;
    // 8192 keys 24.0 -> 23.1; splits of one tile, context 1024: 8.2 -> 9.0).
    // Sixteen waves, the surplus ones only staging: each thread then stages
    // a quarter of a tile instead of half and the kernel needs 124 VGPRs
    // instead of 152 (32 sequences 120.0 -> 103.6 us, 8192 keys 22.1 -> 19.4)
    const int tps = (max_tiles + splits - 1) / splits;
    const bool halves = upb <= 4 && tps >= 2;
    const dim3 grid(n_kv * splits, n_seqs);
    if (halves && tps <= 8 && !bkv) {  // splits of a few tiles: the double-buffered form
      hipLaunchKernelGGL((k_attn_staged<D>), grid, dim3(1024), 0, s, q_hi, q_lo, kv, kv_tiles, part_o, part_ml, o_hi,
                         o_lo, block, n_q, n_kv, splits, scale, st);
      e = hipSuccess;
    } else if (halves) {
      e = attention_tiles<D, false, 1, true>(16, grid, q_hi, q_lo, kv, kv_tiles, bkv, n_seqs, part_o, part_ml, o_hi,
                                             o_lo, block, n_q, n_kv, splits, scale, st, 0, s);
    } else {
      e = attention_tiles<D, false, 1, false>(upb, grid, q_hi, q_lo, kv, kv_tiles, bkv, n_seqs, part_o, part_ml, o_hi,
                                              o_lo, block, n_q, n_kv, splits, scale, st, 0, s);
    }
  }
  if (e != hipSuccess) return e;
  if (splits > 1) {
    // the merge loads every split at once: the smallest instantiation that
    // holds them (each unused slot still costs a shuffle and a select)
    static_assert(kMaxSplits == 64, "merge instantiations cover up to 64 splits");
    const dim3 grid(n_q * ((block + 15) / 16) * 4, n_seqs), blk(256);
    if (splits <= 4)
      hipLaunchKernelGGL((k_attn_merge<D, 4>), grid, blk, 0, s, part_o, part_ml, o_hi, o_lo, block, n_q, splits, st);
    else if (splits <= 8)
      hipLaunchKernelGGL((k_attn_merge<D, 8>), grid, blk, 0, s, part_o, part_ml, o_hi, o_lo, block, n_q, splits, st);
    else if (splits <= 16)
      hipLaunchKernelGGL((k_attn_merge<D, 16>), grid, blk, 0, s, part_o, part_ml, o_hi, o_lo, block, n_q, splits, st);
    else if (splits <= 24)
      hipLaunchKernelGGL((k_attn_merge<D, 24>), grid, blk, 0, s, part_o, part_ml, o_hi, o_lo, block, n_q, splits, st);
    else if (splits <= 32)
      hipLaunchKernelGGL((k_attn_merge<D, 32>), grid, blk, 0, s, part_o, part_ml, o_hi, o_lo, block, n_q, splits, st);
    else if (splits <= 48)
      hipLaunchKernelGGL((k_attn_merge<D, 48>), grid, blk, 0, s, part_o, part_ml, o_hi, o_lo, block, n_q, splits, st);
    else
      hipLaunchKernelGGL((k_attn_merge<D, 64>), grid, blk, 0, s, part_o, part_ml, o_hi, o_lo, block, n_q, splits, st);
  }
  return hipGetLastError();
}

// Grouped launches serve two query heads per wave (each K / V fragment read
// from LDS feeds both; four heads per wave spill registers); one-block
// launches, which are latency-bound at decode sizes, keep one head per wave.
int attention_heads_per_wave(int n_q, int n_kv, bool grouped) {
  const int G = n_q / n_kv;
  return grouped && G % 2 == 0 ? 2 : 1;
}

int attention_group_size(int n_q, int n_kv, int block) {
  const int hpw = attention_heads_per_wave(n_q, n_kv, true);
  const int upb = (n_q / n_kv / hpw) * ((block + 15) / 16);
  // waves serving two heads each hold twice the fragments: at most eight of
  // them per workgroup (sixteen leave 128 registers a wave and spill)
  const int gs = (hpw == 2 ? 8 : 16) / (upb > 0 ? upb : 1);
  return gs < 1 ? 1 : (gs > kAttnGroup ? kAttnGroup : gs);
}

hipError_t launch_attention(const u16* q_hi, const u16* q_lo, const u16* kv_cache, int64_t kv_tiles,
                            const u16* blk_kv, float* part_o, float* part_ml, u16* o_hi, u16* o_lo, int n_seqs,
                            int block, int n_q, int n_kv, int head_dim, int splits, int max_tiles,
                            const SeqTable& st, const AttnGroups* groups, hipStream_t s) {
  if (block > kTileKeys) return hipErrorInvalidValue;
  if (groups && (!blk_kv || groups->n < 1 || groups->n > kMaxSeqs)) return hipErrorInvalidValue;
  if (head_dim == 128)
    return attention_dispatch<128>(q_hi, q_lo, kv_cache, kv_tiles, blk_kv, part_o, part_ml, o_hi, o_lo, n_seqs,
                                   block, n_q, n_kv, splits, max_tiles, st, groups, s);
  if (head_dim == 64)
    return attention_dispatch<64>(q_hi, q_lo, kv_cache, kv_tiles, blk_kv, part_o, part_ml, o_hi, o_lo, n_seqs,
                                  block, n_q, n_kv, splits, max_tiles, st, groups, s);
  return hipErrorInvalidValue;
}

// One thread per 16-byte chunk of the packed layout (see packed_elems): the
// 1 KB block (tile t, k-step s) goes to block t K/32 + s tile-major or
// s n_tiles + t k-major.
template <int MAP>
__global__ __launch_bounds__(256) void k_pack_weights(GemmArgs g, u16* __restrict__ dst) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int S = g.K / 32;
  if (idx >= (size_t)g.n_tiles * S * 64) return;
  const int lane = (int)(idx % 64), c = lane & 15, q = lane >> 4;
  const size_t ts = idx / 64;
  const int s = (int)(ts % S), t = (int)(ts / S);
  const u16* src = weight_row<MAP>(g.w, g.ep, t, c, g.K) + 32 * s + 8 * q;
  const size_t blk = g.pk_kmajor ? (size_t)s * g.n_tiles + t : ts;
  *reinterpret_cast<u32x4*>(dst + (blk * 64 + lane) * 8) = *reinterpret_cast<const u32x4*>(src);
}

hipError_t launch_pack_weights(const GemmArgs& g, u16* dst, hipStream_t s) {
  if (g.K % 32 || g.n_tiles < 1) return hipErrorInvalidValue;
  const size_t chunks = (size_t)g.n_tiles * (g.K / 32) * 64;
  const dim3 grid((unsigned)((chunks + 255) / 256));
  switch (g.map) {
    case MAP_PLAIN: hipLaunchKernelGGL(k_pack_weights<MAP_PLAIN>, grid, dim3(256), 0, s, g, dst); break;
    case MAP_SWIGLU: hipLaunchKernelGGL(k_pack_weights<MAP_SWIGLU>, grid, dim3(256), 0, s, g, dst); break;
    case MAP_QKV: hipLaunchKernelGGL(k_pack_weights<MAP_QKV>, grid, dim3(256), 0, s, g, dst); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int argmax_parts(int n_tiles, int Mp) {
  if (Mp <= 32) return n_tiles / gemm_plan(n_tiles, 0, Mp, false).nc;
  int nm;
  if (const int tail = lm_head_tail(n_tiles, Mp, &nm)) return nm + tail;
  const int tw = lm_head_bn(n_tiles, Mp) / 16;  // MFMA tiles per workgroup column tile
  return (n_tiles + tw - 1) / tw;
}

// One workgroup per block tile; thread t covers slot-major elements of the
// pad slots of all four planes.
__global__ __launch_bounds__(256) void k_clear_block_pad(u16* __restrict__ bkv, int d, int block) {
  u16* tile = bkv + (size_t)blockIdx.x * 4 * kTileKeys * d;
  const int pad = kTileKeys - block, per = pad * d;  // pad elements per plane
  for (int e = threadIdx.x; e < 4 * per; e += 256) {
    const int plane = e / per, w = e % per;
    const int slot = block + w / d, col = w % d;
    // K planes [slot][d]; V planes [d][slot]
    const size_t off = plane < 2 ? (size_t)slot * d + col : (size_t)col * kTileKeys + slot;
    tile[(size_t)plane * kTileKeys * d + off] = 0;
  }
}

hipError_t launch_clear_block_pad(u16* blk_kv, int n_blocks, int n_kv, int head_dim, int block, hipStream_t s) {
  if (block > kTileKeys || n_blocks < 1) return hipErrorInvalidValue;
  if (block == kTileKeys) return hipSuccess;
  hipLaunchKernelGGL(k_clear_block_pad, dim3(n_blocks * n_kv), dim3(256), 0, s, blk_kv, head_dim, block);
  return hipGetLastError();
}

hipError_t launch_argmax_reduce(const unsigned long long* part, int n_parts, int Mp, int n_seqs,
                                int block, int32_t* draft, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_reduce, dim3(n_seqs * (block - 1)), dim3(256), 0, s, part, n_parts, Mp,
                     block, draft);
  return hipGetLastError();
}

size_t verify_scratch_bytes(int n, int block, int vocab) {
  const size_t C = verify_chunks(vocab), CR = verify_rchunks(vocab);
  const size_t lse = (size_t)n * block * C * sizeof(Lse4);
  return lse + (size_t)n * sizeof(VerifyPos) + (size_t)n * CR * (sizeof(double) + sizeof(int)) + 64;
}

hipError_t launch_verify_sample(const int32_t* draft, const float* q_logits, const float* p_logits, int n,
                                int block, int vocab, double temp, unsigned long long seed, void* scratch,
                                int32_t* accept, int32_t* next_token, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (block < 2 || block > 1024 || vocab < 1 || vocab > kVerifyMaxVocab) return hipErrorInvalidValue;
  const int C = verify_chunks(vocab), CR = verify_rchunks(vocab);
  Lse4* part = (Lse4*)scratch;
  VerifyPos* vp = (VerifyPos*)(part + (size_t)n * block * C);
  double* cand_v = (double*)(vp + n);
  int* cand_i = (int*)(cand_v + (size_t)n * CR);
  const double inv_t = 1.0 / temp;
  hipLaunchKernelGGL(k_verify_lse, dim3(n * block * C), dim3(256), 0, s, q_logits, p_logits, block, vocab, C, inv_t,
                     part);
  hipLaunchKernelGGL(k_verify_keep, dim3(n), dim3(1024), 0, s, draft, q_logits, p_logits, block, vocab, C, inv_t,
                     seed, part, vp, accept);
  hipLaunchKernelGGL(k_verify_sample, dim3(n * CR), dim3(256), 0, s, q_logits, p_logits, block, vocab, CR, inv_t,
                     seed, vp, cand_v, cand_i);
  hipLaunchKernelGGL(k_verify_final, dim3((n + 3) / 4), dim3(256), 0, s, cand_v, cand_i, n, CR, vocab, next_token);
  return hipGetLastError();
}

hipError_t launch_accept(const int32_t* draft, const int32_t* target, int n, int block,
                         int32_t* accept, int32_t* next_anchor, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_accept, dim3((n + 3) / 4), dim3(256), 0, s, draft, target, n, block, accept,
                     next_anchor);
  return hipGetLastError();
}

}  // namespace dflash
