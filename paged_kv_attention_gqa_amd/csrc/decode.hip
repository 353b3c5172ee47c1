// Paged GQA decode for gfx950 (MI355X): Hq = 32, Hkv = 4, head_dim = 128,
// bf16 q/K/V, fp32 accumulation, base-2 LSE.
//
// What is computed follows kernelindex.com, "flashinfer gemini-2.5-pro /
// triton h7ykt0" (gqa_paged_decode_h32_kv4_d128_ps1, steps 4-9): gather each
// token's K and V row through the CSR page list, scaled q.k scores, online
// softmax, P.V, then out = acc / l and lse = log2 of the exp-sum. The split into
// chunks with normalised fp32 partials and an LSE merge follows the vLLM fork
// qsa.py (_qsa_sparse_paged_gqa_splitk_kernel, _qsa_merge_splitk_kernel).
// Pages of several tokens found through a block table follow the FlagGems
// flash_mla_with_kvcache page (_dense_decode_kernel): token t of a sequence is
// slot t % page_size of page table[t / page_size]. Both forms reduce to one
// pool row index per token, (page << log2(page_size)) | slot, which is all the
// kernel below uses; page sizes are powers of two.
//
// Design (gfx950, wave64):
// * One workgroup per worker of the plan: a cost-balanced run of the batch's tokens,
//   as a list of (sequence, token range) segments. Wave w handles KV head w
//   and its 8 query heads and walks each segment in tiles of 32 tokens.
// * Both contractions run on v_mfma_f32_16x16x32_bf16 (MfmaEngine, the
//   default; Dot2Engine below runs them on the vector ALU instead), the 8
//   query heads padded to 16 MFMA columns:
//     S^T[tok, h] = K[tok, :] . Q[h, :]        A = K rows as loaded, B = Q^T
//     O^T[d, h]  += V^T[d, tok] . P^T[tok, h]  A = V^T read back from LDS, B = P^T
//   The S^T accumulator leaves lane (r, c) = (lane % 16, lane / 16) with head r
//   and tokens 16*mb + 4c + i, which is exactly the token set the P^T operand
//   of lane (r, c) needs, so P never crosses lanes. The MFMA only needs A and B
//   to agree on the order of the contracted index, so neither K nor P is
//   shuffled.
// * K/V rows are gathered straight into registers: lane (r, c) reads bytes
//   [64x + 16c, +16) of the 256-byte (page, KV head) row of token 16*mb + r,
//   so one load instruction covers 64 contiguous bytes of 16 rows.
// * V is written to LDS row-major (288-byte padded rows) and read back as the
//   transposed A operand (8 tokens of one dim per lane) with the
//   transposing LDS load ds_read_b64_tr_b16, two per 16-dim block.
// * Loads are software-pipelined one tile ahead, page ids two tiles ahead
//   (for a CSR page list staged through a 128-byte LDS slot per wave: one
//   coalesced read of a tile's 32 ids, then two LDS reads per lane; the
//   vector-ALU engine issues loads earlier and keeps ids in registers, see
//   process_segment);
//   out-of-range tokens of the last tile re-read the item's last page, which
//   keeps every load unconditional, and get score -inf, i.e. weight exactly 0.
// * Scores are scaled by sm_scale*log2(e) in fp32 and exponentiated with
//   exp2; the running max is reduced across the 4 lane rows with the
//   cross-lane swaps v_permlane16_swap / v_permlane32_swap (vector ALU, no
//   LDS), the running sum is kept per lane and reduced once at the end.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "lanes.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = kHq / kHkv;      // query heads per KV head
constexpr int kTileTok = 32;            // tokens per wave per step
constexpr int kRowU16 = kHeadDim + 16;  // LDS row of one token's V: 256 B + 32 B pad
constexpr int kThreads = 64 * kHkv;
constexpr int kPipeTiles = 2;           // register tile buffers per wave
constexpr float kNegInf = -__builtin_huge_valf();

struct Tile {
  u32x4 k[2][4];  // [mb][x]: bytes [64x + 16c, +16) of the K row of token 16*mb + r
  u32x4 v[2][4];
};

struct Softmax {
  f32x4 acc[8];   // O^T blocks: acc[db][i] = O[head r][16*db + 4c + i]
  float m;        // running max of the log2-domain scores (equal on the 4 lane rows)
  float l;        // this lane's share of the running exp-sum
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ void load_tile(Tile& t, const uint16_t* __restrict__ k_pool,
                                          const uint16_t* __restrict__ v_pool, int32_t page0,
                                          int32_t page1, int g, int c) {
  const int64_t r0 = (static_cast<int64_t>(page0) * kHkv + g) * kHeadDim + c * 8;
  const int64_t r1 = (static_cast<int64_t>(page1) * kHkv + g) * kHeadDim + c * 8;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    t.k[0][x] = *reinterpret_cast<const u32x4*>(k_pool + r0 + x * 32);
    t.k[1][x] = *reinterpret_cast<const u32x4*>(k_pool + r1 + x * 32);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    t.v[0][x] = *reinterpret_cast<const u32x4*>(v_pool + r0 + x * 32);
    t.v[1][x] = *reinterpret_cast<const u32x4*>(v_pool + r1 + x * 32);
  }
}

// Orders this wave's LDS writes before its later LDS reads (and the reverse).
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// First half of a tile: scores of the 32 tokens against the (padded) 16
// heads, the online-softmax update, and the tile's V rows into LDS. After it
// the tile's registers are free; pb holds P for compute_back.
__device__ __forceinline__ void compute_front(const Tile& t, int t0, int n, const u32x4 (&qf)[4],
                                              float scale_log2, int r, int c, uint16_t* lw,
                                              Softmax& st, bf16x8& pb) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
  f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k[0][x]), as_bf16x8(qf[x]), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k[1][x]), as_bf16x8(qf[x]), s1, 0, 0, 0);
  }
  // p[4*mb + i] belongs to token t0 + 16*mb + 4c + i.
  float p[8];
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = t0 + 4 * c + i;
    p[i] = (tok < n) ? s0[i] * scale_log2 : kNegInf;
    p[4 + i] = (tok + 16 < n) ? s1[i] * scale_log2 : kNegInf;
    mx = fmaxf(mx, fmaxf(p[i], p[4 + i]));
  }
  mx = max_xor32(max_xor16(mx));
  const float m_new = fmaxf(st.m, mx);   // finite: every tile holds a valid token
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __builtin_amdgcn_exp2f(p[j] - m_new);
    psum += p[j];
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
#pragma unroll
  for (int db = 0; db < 8; ++db) st.acc[db] *= alpha;

  // V rows to LDS (row-major, padded rows).
  lds_wave_sync();
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      *reinterpret_cast<u32x4*>(lw + (16 * mb + r) * kRowU16 + 32 * x + 8 * c) = t.v[mb][x];
    }
  }
  lds_wave_sync();

#pragma unroll
  for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(p[j]);
}

// Second half: O^T += V^T P^T from the LDS copy of the tile's V rows.
__device__ __forceinline__ void compute_back(const bf16x8& pb, int r, int c, const uint16_t* lw,
                                             Softmax& st) {
  // A operand of block db: V[token 16*(j/4) + 4c + j%4][16*db + r], j = 0..7,
  // read with the transposing LDS load: within each 16-lane group it gives
  // lane i element i%4 of the 8-byte chunks addressed by lanes 4j + i/4, so
  // lane (r, c) points at token 4c + r/4 (and 16 more), dims 16 db + 4 (r%4).
  const uint16_t* vrow0 = lw + (4 * c + (r >> 2)) * kRowU16 + 4 * (r & 3);
  const uint16_t* vrow1 = vrow0 + 16 * kRowU16;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vrow0 + 16 * db));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vrow1 + 16 * db));
    const u32x4 a = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                     __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), pb, st.acc[db], 0, 0, 0);
  }
}

// The two contraction engines a segment can run on. Each keeps the wave's
// query heads and softmax state, consumes tiles as the pipeline in
// process_segment delivers them, and writes the segment's result.
//
// Each tile is taken in two calls: front() (scores, softmax, V rows into LDS)
// after which the tile's registers may be reloaded, and back() (P.V from
// LDS).
//
// MfmaEngine: both contractions on v_mfma_f32_16x16x32_bf16 (compute_front,
// compute_back).
struct MfmaEngine {
  static constexpr int kIdSlotU16 = kTileTok * kRowU16;       // after the V tile: 32 page ids
  static constexpr int kWaveLdsU16 = kIdSlotU16 + 2 * kTileTok;
  static constexpr int kWavesPerEu = 2;
  static constexpr bool kEarlyLoads = false;
  u32x4 qf[4];
  Softmax st;
  bf16x8 pb;   // P of the tile between front() and back()

  // Q as the B operand: lane (r, c) holds q[head r][32x + 8c, +8) for k-step
  // x. The 8 padding columns (r >= kGroup) repeat heads r - kGroup: their
  // scores and outputs are computed and never stored.
  __device__ __forceinline__ void begin(const uint16_t* __restrict__ q, int b, int g, int r, int c) {
    const uint16_t* qh =
        q + (static_cast<int64_t>(b) * kHq + g * kGroup + (r & (kGroup - 1))) * kHeadDim + 8 * c;
#pragma unroll
    for (int x = 0; x < 4; ++x) qf[x] = *reinterpret_cast<const u32x4*>(qh + 32 * x);
#pragma unroll
    for (int db = 0; db < 8; ++db) st.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = kNegInf;
    st.l = 0.f;
  }

  __device__ __forceinline__ void front(const Tile& t, int t0, int n, float scale_log2, int r,
                                        int c, uint16_t* lw) {
    compute_front(t, t0, n, qf, scale_log2, r, c, lw, st, pb);
  }

  __device__ __forceinline__ void back(int r, int c, const uint16_t* lw) {
    compute_back(pb, r, c, lw, st);
  }

  __device__ __forceinline__ void finish(int b, int g, int slot, int r, int c,
                                         uint16_t* __restrict__ out, float* __restrict__ lse,
                                         float* __restrict__ part_o, float* __restrict__ part_lse) {
    const int head = g * kGroup + r;   // a real query head only for r < kGroup
    const float l_tot = sum_xor32(sum_xor16(st.l));
    const float inv = 1.0f / l_tot;
    const float lse2 = st.m + __log2f(l_tot);
    if (r < kGroup) {
      if (slot < 0) {
        uint16_t* o = out + (static_cast<int64_t>(b) * kHq + head) * kHeadDim + 4 * c;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const f32x4 v = st.acc[db] * inv;
          const u32x2 w = {static_cast<uint32_t>(bf16_bits(v[0])) |
                               (static_cast<uint32_t>(bf16_bits(v[1])) << 16),
                           static_cast<uint32_t>(bf16_bits(v[2])) |
                               (static_cast<uint32_t>(bf16_bits(v[3])) << 16)};
          *reinterpret_cast<u32x2*>(o + 16 * db) = w;
        }
        if (c == 0) lse[b * kHq + head] = lse2;
      } else {
        float* o = part_o + (static_cast<int64_t>(slot) * kHq + head) * kHeadDim + 4 * c;
#pragma unroll
        for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(o + 16 * db) = st.acc[db] * inv;
        if (c == 0) part_lse[static_cast<int64_t>(slot) * kHq + head] = lse2;
      }
    }
  }
};

// Dot2Engine: both contractions on the vector ALU with v_dot2c_f32_bf16 (two
// bf16 products summed into an fp32 accumulator per lane and instruction),
// over the same tiles and the same K/V register layout as the MFMA engine.
// * Scores: lane (r, c) holds dims {32x + 8c .. +8 | x < 4} of tokens r and
//   16 + r, and forms their partial dot products with all 8 heads (q is read
//   from the wave's LDS copy, 16 lanes sharing each 16-byte read). The four
//   lanes of a token (c = 0..3) then sum their partials in two halving steps
//   (split_sum_xor32, split_sum_xor16), after which lane (r, c) holds the full
//   scores of tokens r and 16 + r for heads 2c and 2c + 1.
// * Softmax: the tile max of a head is reduced over the 16 lanes of its row
//   (DPP), and the 8 heads' maxima are shared with every lane by cross-lane
//   swaps, so every lane can rescale its accumulators of all 8 heads; the
//   running sum is kept per lane and reduced at the end of the segment.
// * P.V: P (bf16) goes to LDS as [token quad][head][4 tokens]; lane (r, c)
//   owns output dims 16c + r and 64 + 16c + r of all 8 heads and reads V^T
//   pairs (two consecutive tokens of one dim) with ds_read_b64_tr_b16, each
//   a dot2 operand against the matching pair of P, which all lanes read at the
//   same LDS address.
struct Dot2Engine {
  static constexpr int kQU16 = kGroup * kHeadDim;   // the wave's q block, row-major by head
  static constexpr int kPU16 = kTileTok * kGroup;   // P of one tile
  static constexpr int kWaveLdsU16 = kTileTok * kRowU16 + kQU16 + kPU16;
  static constexpr int kIdSlotU16 = -1;   // the early-load pipeline keeps page ids in registers
  static constexpr int kWavesPerEu = 2;
  static constexpr bool kEarlyLoads = true;
  u32x4 qa, qb;          // bytes [32 lane, +32) of the q block, until they go to LDS
  float acc[kGroup][2];  // O[head h][dim 16c + r], O[head h][dim 64 + 16c + r]
  float m_all[kGroup];   // running max of each head (the same in every lane)
  float m_own[2];        // running max of heads 2c, 2c + 1 (equal to m_all's)
  float l_own[2];        // this lane's share of their exp-sums

  __device__ __forceinline__ void begin(const uint16_t* __restrict__ q, int b, int g, int r, int c) {
    const int lane = 16 * c + r;
    const uint16_t* qg = q + (static_cast<int64_t>(b) * kHq + g * kGroup) * kHeadDim + 16 * lane;
    qa = *reinterpret_cast<const u32x4*>(qg);
    qb = *reinterpret_cast<const u32x4*>(qg + 8);
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      acc[h][0] = 0.f;
      acc[h][1] = 0.f;
      m_all[h] = kNegInf;
    }
    m_own[0] = m_own[1] = kNegInf;
    l_own[0] = l_own[1] = 0.f;
  }

  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
  }

  // The 8 heads' values of a per-row quantity (v[j] of row c belongs to head
  // 2c + j) in every lane: out[2c' + j] = row c' value j.
  static __device__ __forceinline__ void share_rows(const float (&v)[2], float (&out)[kGroup]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const lane_u32x2 p16 = pair_xor16(v[j]);   // rows c & ~1, c | 1
      const unsigned lo = p16[0], hi = p16[1];
      const lane_u32x2 a = pair_xor32(__builtin_bit_cast(float, lo));   // rows 0, 2
      const lane_u32x2 e = pair_xor32(__builtin_bit_cast(float, hi));   // rows 1, 3
      const unsigned a0 = a[0], a1 = a[1], e0 = e[0], e1 = e[1];
      out[0 + j] = __builtin_bit_cast(float, a0);
      out[2 + j] = __builtin_bit_cast(float, e0);
      out[4 + j] = __builtin_bit_cast(float, a1);
      out[6 + j] = __builtin_bit_cast(float, e1);
    }
  }

  __device__ __forceinline__ void front(const Tile& t, int t0, int n, float scale_log2, int r,
                                        int c, uint16_t* lw) {
    uint16_t* lq = lw + kTileTok * kRowU16;
    uint16_t* lp = lq + kQU16;
    if (t0 == 0) {   // the segment's first tile: q to LDS
      lds_wave_sync();
      *reinterpret_cast<u32x4*>(lq + 16 * (16 * c + r)) = qa;
      *reinterpret_cast<u32x4*>(lq + 16 * (16 * c + r) + 8) = qb;
    }
    lds_wave_sync();

    // Partial scores of tokens r (mb 0) and 16 + r (mb 1) over this lane's
    // dims, one 8-dim slice at a time: the slice's q reads (one per head)
    // all leave before any is used, so a slice costs one LDS round trip.
    float s[2][kGroup];
#pragma unroll
    for (int h = 0; h < kGroup; ++h) s[0][h] = s[1][h] = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      __builtin_amdgcn_sched_barrier(0);
      u32x4 qv[kGroup];
#pragma unroll
      for (int h = 0; h < kGroup; ++h)
        qv[h] = *reinterpret_cast<const u32x4*>(lq + h * kHeadDim + 32 * x + 8 * c);
#pragma unroll
      for (int h = 0; h < kGroup; ++h) asm volatile("" : "+v"(qv[h]));
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t qe = qv[h][e];
          const uint32_t k0 = t.k[0][x][e], k1 = t.k[1][x][e];
          s[0][h] = dot2(k0, qe, s[0][h]);
          s[1][h] = dot2(k1, qe, s[1][h]);
        }
      }
#pragma unroll
      for (int h = 0; h < kGroup; ++h) asm volatile("" : "+v"(s[0][h]), "+v"(s[1][h]));
    }
    // Sum over the token's four lanes: rows c >> 1 == 0 keep heads 0-3, then
    // rows with c & 1 == 0 keep the first two of those: lane (r, c) ends
    // with heads 2c and 2c + 1.
    float s4[2][4], sc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int h = 0; h < 4; ++h) s4[mb][h] = split_sum_xor32(s[mb][h], s[mb][h + 4]);
#pragma unroll
      for (int j = 0; j < 2; ++j) sc[mb][j] = split_sum_xor16(s4[mb][j], s4[mb][j + 2]);
    }

    // Online softmax in the log2 domain.
    float a[2][2], mx[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      a[0][j] = (t0 + r < n) ? sc[0][j] * scale_log2 : kNegInf;
      a[1][j] = (t0 + 16 + r < n) ? sc[1][j] * scale_log2 : kNegInf;
      mx[j] = row_max16(fmaxf(a[0][j], a[1][j]));   // finite: every tile holds a valid token
    }
    float mx_all[kGroup];
    share_rows(mx, mx_all);
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const float m_new = fmaxf(m_all[h], mx_all[h]);
      const float alpha = __builtin_amdgcn_exp2f(m_all[h] - m_new);
      m_all[h] = m_new;
      acc[h][0] *= alpha;
      acc[h][1] *= alpha;
    }
    float p[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float m_new = fmaxf(m_own[j], mx[j]);
      const float alpha = __builtin_amdgcn_exp2f(m_own[j] - m_new);
      m_own[j] = m_new;
      p[0][j] = __builtin_amdgcn_exp2f(a[0][j] - m_new);
      p[1][j] = __builtin_amdgcn_exp2f(a[1][j] - m_new);
      l_own[j] = l_own[j] * alpha + (p[0][j] + p[1][j]);
    }

    // V rows and P to LDS.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        *reinterpret_cast<u32x4*>(lw + (16 * mb + r) * kRowU16 + 32 * x + 8 * c) = t.v[mb][x];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        lp[((4 * mb + (r >> 2)) * kGroup + 2 * c + j) * 4 + (r & 3)] = bf16_bits(p[mb][j]);
    }
    lds_wave_sync();
  }

  __device__ __forceinline__ void back(int r, int c, const uint16_t* lw) {
    const uint16_t* lp = lw + kTileTok * kRowU16 + kQU16;
    // P.V over the 8 token quads: lane (r, c) reads tokens 4qd .. 4qd + 3 of
    // dims 16c + r and 64 + 16c + r (the transposing read: lane 4j + i of a
    // row addresses token 4qd + j, dims 16c + 4i .. +4).
    const uint16_t* vb = lw + (r >> 2) * kRowU16 + 4 * (r & 3) + 16 * c;
#pragma unroll
    for (int q2 = 0; q2 < kTileTok / 8; ++q2) {
      // two quads per LDS round trip: their 4 V^T reads and 8 P reads leave
      // before any is used
      __builtin_amdgcn_sched_barrier(0);
      u32x2 vt[2][2];
      u32x4 pq[2][kGroup / 2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qd = 2 * q2 + u;
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
          vt[u][hi] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                         (__attribute__((address_space(3))) i16x4*)(vb + 4 * qd * kRowU16 + 64 * hi)));
#pragma unroll
        for (int hp = 0; hp < kGroup / 2; ++hp)
          pq[u][hp] = *reinterpret_cast<const u32x4*>(lp + (qd * kGroup + 2 * hp) * 4);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        asm volatile("" : "+v"(vt[u][0]), "+v"(vt[u][1]));
#pragma unroll
        for (int hp = 0; hp < kGroup / 2; ++hp) asm volatile("" : "+v"(pq[u][hp]));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t v00 = vt[u][0][0], v01 = vt[u][0][1], v10 = vt[u][1][0], v11 = vt[u][1][1];
#pragma unroll
        for (int hp = 0; hp < kGroup / 2; ++hp) {
          // heads 2hp, 2hp + 1: P pairs (4qd, 4qd + 1), (4qd + 2, 4qd + 3) each
          const uint32_t p0 = pq[u][hp][0], p1 = pq[u][hp][1], p2 = pq[u][hp][2], p3 = pq[u][hp][3];
          acc[2 * hp][0] = dot2(v01, p1, dot2(v00, p0, acc[2 * hp][0]));
          acc[2 * hp][1] = dot2(v11, p1, dot2(v10, p0, acc[2 * hp][1]));
          acc[2 * hp + 1][0] = dot2(v01, p3, dot2(v00, p2, acc[2 * hp + 1][0]));
          acc[2 * hp + 1][1] = dot2(v11, p3, dot2(v10, p2, acc[2 * hp + 1][1]));
        }
      }
      // The products are done here: without this the compiler sinks them to
      // the accumulators' next use in the following tile, keeping every P
      // read of this tile live across the next tile's loads.
#pragma unroll
      for (int h = 0; h < kGroup; ++h) asm volatile("" : "+v"(acc[h][0]), "+v"(acc[h][1]));
    }
  }

  __device__ __forceinline__ void finish(int b, int g, int slot, int r, int c,
                                         uint16_t* __restrict__ out, float* __restrict__ lse,
                                         float* __restrict__ part_o, float* __restrict__ part_lse) {
    float l_row[2], inv_own[2], inv_all[kGroup];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      l_row[j] = row_sum16(l_own[j]);
      inv_own[j] = 1.0f / l_row[j];
    }
    share_rows(inv_own, inv_all);
    const int64_t head0 = static_cast<int64_t>(slot < 0 ? b : slot) * kHq + g * kGroup;
    const int d0 = 16 * c + r;
    if (slot < 0) {
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        uint16_t* o = out + (head0 + h) * kHeadDim + d0;
        o[0] = bf16_bits(acc[h][0] * inv_all[h]);
        o[64] = bf16_bits(acc[h][1] * inv_all[h]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        float* o = part_o + (head0 + h) * kHeadDim + d0;
        o[0] = acc[h][0] * inv_all[h];
        o[64] = acc[h][1] * inv_all[h];
      }
    }
    if (r == 0) {
      float* dst = slot < 0 ? lse : part_lse;
#pragma unroll
      for (int j = 0; j < 2; ++j) dst[head0 + 2 * c + j] = m_own[j] + __log2f(l_row[j]);
    }
  }
};

// Pool row (page * page_size + slot) of token j of a segment.
template <bool kTable>
struct TokenRows;

// CSR page list, page size 1: the row is the listed page.
template <>
struct TokenRows<false> {
  const int32_t* ids;   // page ids of the segment's tokens
  __device__ TokenRows(const KvAddressing& a, int b, int lo, int seq_offset)
      : ids(a.ids + seq_offset + lo) {}
  __device__ __forceinline__ int32_t fetch(int j) const { return ids[j]; }
  __device__ __forceinline__ int32_t row_of(int32_t fetched, int) const { return fetched; }
  __device__ __forceinline__ int32_t operator()(int j) const { return row_of(fetch(j), j); }
};

// Block table: token t = lo + j of sequence b is slot t % ps of page row[t / ps].
template <>
struct TokenRows<true> {
  const int32_t* row;   // the sequence's block-table row
  int lo, shift, mask;
  __device__ TokenRows(const KvAddressing& a, int b, int lo_, int)
      : row(a.ids + static_cast<int64_t>(b) * a.table_stride), lo(lo_), shift(a.page_shift),
        mask((1 << a.page_shift) - 1) {}
  __device__ __forceinline__ int32_t fetch(int j) const { return row[(lo + j) >> shift]; }
  __device__ __forceinline__ int32_t row_of(int32_t page, int j) const {
    return (page << shift) | ((lo + j) & mask);
  }
  __device__ __forceinline__ int32_t operator()(int j) const { return row_of(fetch(j), j); }
};

// Decodes the n > 0 tokens of a segment of sequence b, whose pool rows `ids`
// gives, with all four waves of the workgroup and writes either the final
// out/lse (slot < 0) or a partial.
template <bool kTable, class Engine>
__device__ __forceinline__ void process_segment(
    const TokenRows<kTable>& ids, int b, int n, int slot, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, uint16_t* lds) {
  const int lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // KV head of this wave
  const int r = lane & 15;
  const int c = lane >> 4;
  const int last = n - 1;

  // The ids of the first two tiles are fetched first: they depend only on
  // the segment's position, so (for a worker's first segment, whose position
  // comes with the kernel arguments) they leave before q, which needs b.
  const int ja0 = min(r, last), ja1 = min(16 + r, last);
  const int jn0 = min(kTileTok + r, last), jn1 = min(kTileTok + 16 + r, last);
  int32_t a0 = ids.fetch(ja0), a1 = ids.fetch(ja1);
  int32_t n0 = ids.fetch(jn0), n1 = ids.fetch(jn1);

  // q of the wave's query heads (every lane loads, so the compiler can count
  // the loads in flight: a masked load made it wait for q before the first
  // K/V loads).
  Engine eng;
  eng.begin(q, b, g, r, c);
  uint16_t* lw = lds + g * Engine::kWaveLdsU16;   // each wave owns its LDS slice

  // Software pipeline over a ring of two register tiles, unrolled over the
  // ring so every buffer index is a constant and the loop body has no early
  // exit; the empty asm statements keep each load group where it is written.
  // Page ids are fetched ahead of the K/V loads they feed and issued before
  // the K/V loads of the tile before, so waiting for ids never waits for
  // younger K/V loads. Loads past the segment re-read its last row (all lanes
  // the same row: one cache line per lane group), and an odd last tile is
  // computed after the loop from the buffer the final iterations loaded.
  //
  // Engine::kEarlyLoads picks where the next loads go out. false: at tile T,
  // load tile T + 1 into the buffer of tile T - 1, then compute T (one tile in
  // flight during the compute; fastest for the short MFMA compute). true:
  // front(T) consumes tile T's registers, tile T + 2 is loaded into them, then
  // back(T) runs while tiles T + 1 and T + 2 are in flight (for the longer
  // vector-ALU compute).
  const int n_tiles = (n + kTileTok - 1) / kTileTok;
  const int n_rounds = n_tiles / kPipeTiles;
  static_assert(kPipeTiles == 2, "the prologue below fills a ring of two tiles");
  Tile ring[kPipeTiles];
  int t0 = 0;
  if constexpr (Engine::kEarlyLoads) {
    const int jc0 = min(2 * kTileTok + r, last), jc1 = min(2 * kTileTok + 16 + r, last);
    int32_t c0 = ids.fetch(jc0), c1 = ids.fetch(jc1);
    // The first two tiles' ids (fetched above) are all in before any K/V
    // load; the third tile's, fetched after q, may still be in flight.
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(n0), "+v"(n1));
    load_tile(ring[0], k_pool, v_pool, ids.row_of(a0, ja0), ids.row_of(a1, ja1), g, c);
    load_tile(ring[1], k_pool, v_pool, ids.row_of(n0, jn0), ids.row_of(n1, jn1), g, c);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(c0), "+v"(c1));
    int32_t next0 = ids.row_of(c0, jc0);
    int32_t next1 = ids.row_of(c1, jc1);
    for (int round = 0; round < n_rounds; ++round) {
#pragma unroll
      for (int k = 0; k < kPipeTiles; ++k) {
        // front of tile T = 2 round + k (ring[k]); fetch the ids of tile
        // T + 3; load tile T + 2 into ring[k]; back of tile T.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        eng.front(ring[k], t0 + kTileTok * k, n, scale_log2, r, c, lw);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        const int tf = t0 + kTileTok * (k + 3);
        const int j0 = min(tf + r, last);
        const int j1 = min(tf + 16 + r, last);
        int32_t f0 = ids.fetch(j0);
        int32_t f1 = ids.fetch(j1);
        load_tile(ring[k], k_pool, v_pool, next0, next1, g, c);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        eng.back(r, c, lw);
        __builtin_amdgcn_sched_barrier(0);
        // The fetched ids stay opaque until the compute above has been
        // issued, so nothing derived from them is scheduled next to their
        // loads (which would make the wave wait for loads it has just issued).
        asm volatile("" : "+v"(f0), "+v"(f1));
        next0 = ids.row_of(f0, j0);
        next1 = ids.row_of(f1, j1);
      }
      t0 += kTileTok * kPipeTiles;
    }
  } else {
    // The first two tiles' ids (fetched above) are all in before any K/V
    // load, so the loop starts with the second tile's rows known and no load
    // pending but the first tile's.
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(n0), "+v"(n1));
    load_tile(ring[0], k_pool, v_pool, ids.row_of(a0, ja0), ids.row_of(a1, ja1), g, c);
    int32_t next0 = ids.row_of(n0, jn0);
    int32_t next1 = ids.row_of(n1, jn1);
    for (int round = 0; round < n_rounds; ++round) {
#pragma unroll
      for (int k = 0; k < kPipeTiles; ++k) {
        // compute tile round * kPipeTiles + k (ring[k]); load the tile after
        // it into the buffer computed last; fetch the ids of the tile after
        // that.
        asm volatile("" ::: "memory");
        const int tf = t0 + kTileTok * (k + kPipeTiles);
        const int j0 = min(tf + r, last);
        const int j1 = min(tf + 16 + r, last);
        int32_t f0, f1 = 0;
        if constexpr (kTable) {
          f0 = ids.fetch(j0);
          f1 = ids.fetch(j1);
        } else {
          // The page list is staged through LDS: lanes 16c + r (c < 2) load
          // the tile's 32 ids in one coalesced 128-byte read (lanes c >= 2
          // repeat it), and after the compute below they go to the wave's
          // id slot, from which every lane reads the two it needs.
          f0 = ids.fetch(min(tf + ((16 * c + r) & 31), last));
        }
        load_tile(ring[(k + kPipeTiles - 1) % kPipeTiles], k_pool, v_pool, next0, next1, g, c);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        eng.front(ring[k], t0 + kTileTok * k, n, scale_log2, r, c, lw);
        eng.back(r, c, lw);
        __builtin_amdgcn_sched_barrier(0);
        // The fetched ids stay opaque until the compute above has been
        // issued, so nothing derived from them is scheduled next to their
        // loads (which would make the wave wait for loads it has just issued).
        if constexpr (kTable) {
          asm volatile("" : "+v"(f0), "+v"(f1));
          next0 = ids.row_of(f0, j0);
          next1 = ids.row_of(f1, j1);
        } else {
          asm volatile("" : "+v"(f0));
          int32_t* slot_ids = reinterpret_cast<int32_t*>(lw + Engine::kIdSlotU16);
          lds_wave_sync();
          if (c < 2) slot_ids[16 * c + r] = f0;
          lds_wave_sync();
          next0 = slot_ids[r];
          next1 = slot_ids[16 + r];
        }
      }
      t0 += kTileTok * kPipeTiles;
    }
  }
  if (n_tiles > n_rounds * kPipeTiles) {
    eng.front(ring[0], t0, n, scale_log2, r, c, lw);
    eng.back(r, c, lw);
  }
  eng.finish(b, g, slot, r, c, out, lse, part_o, part_lse);
}

// One workgroup per worker: it walks its segments in order. The first
// kFirstArgWorkers workers find where their first segment's ids start in the
// kernel arguments (CSR: (kv_indptr[b] + tok_begin, 0, n); block table: (b,
// tok_begin, n); n = 0 if the worker has no segment), so its id loads leave
// one memory round trip earlier than the worker's record, which still
// supplies b, the slot and the segment range.
template <bool kTable, class Engine>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Engine::kWavesPerEu))) void decode_partial_kernel(
    const int32_t* __restrict__ workers, const int32_t* __restrict__ segments,
    const FirstSegments firsts, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool, KvAddressing addr,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kHkv * Engine::kWaveLdsU16];
  const int w = blockIdx.x;
  const bool first_in_args = w < kFirstArgWorkers;
  // Read (clamped in range) before any branch, so the loads go out together
  // with the other argument loads.
  const int wf = min(w, kFirstArgWorkers - 1);
  int f0 = firsts.v[3 * wf], f1 = firsts.v[3 * wf + 1], n = firsts.v[3 * wf + 2];
  int wofs = 8 * w;
  asm volatile("" : "+s"(f0), "+s"(f1), "+s"(n), "+s"(wofs));
  const int32_t* wrec = workers + wofs;   // first segment inline, then its range
  if (first_in_args) {
    if (n > 0) {
      const TokenRows<kTable> ids(addr, kTable ? f0 : 0, f1, kTable ? 0 : f0);
      process_segment<kTable, Engine>(ids, wrec[0], n, wrec[3], q, k_pool, v_pool, scale_log2, out, lse,
                              part_o, part_lse, lds);
    }
  }
  const int s_begin = wrec[5];
  const int s_end = wrec[6];
  for (int s = first_in_args ? s_begin + 1 : s_begin; s < s_end; ++s) {
    const int32_t* seg = s == s_begin ? wrec : segments + 8 * s;
    const int lo = seg[1];
    const int n = seg[2] - lo;
    if (n > 0) {
      const TokenRows<kTable> ids(addr, seg[0], lo, seg[4]);
      process_segment<kTable, Engine>(ids, seg[0], n, seg[3], q, k_pool, v_pool, scale_log2, out, lse,
                              part_o, part_lse, lds);
    }
  }
}

// One wave per (merge record, query head), four heads per workgroup. Lane
// (p, e) = (lane / 16, lane % 16) owns dims [8e, 8e + 8) of the partials
// i = 4j + p. The partials are taken in rounds of 4J: every load of a round
// (one LSE per lane, two 16-byte loads per lane and partial) is issued before
// any is used, and the round is folded into the running result against a
// running maximum, so a sequence cut into up to ~120 pieces costs one round
// trip to memory. The four lane groups are summed at the end in a fixed
// order, so the result does not depend on timing.
template <int J>
__device__ __forceinline__ void merge_round(const float* part_o, const float* part_lse, int first,
                                            int k,
                                            int i0, int h, int lane, float& top, float& den,
                                            f32x4 (&acc)[2]) {
  const int p = lane >> 4;
  const int e = lane & 15;
  // LSE of partial i0 + lane (-inf past the end).
  const int il = i0 + lane;
  float li = part_lse[static_cast<int64_t>(first + min(il, k - 1)) * kHq + h];
  f32x4 o[J][2];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = min(i0 + 4 * j + p, k - 1);
    const float* src = part_o + (static_cast<int64_t>(first + i) * kHq + h) * kHeadDim + 8 * e;
    o[j][0] = *reinterpret_cast<const f32x4*>(src);
    o[j][1] = *reinterpret_cast<const f32x4*>(src + 4);
  }
  // Every load of the round is issued before the first of these statements
  // (they clobber memory), and every use comes after its value passes one.
  asm volatile("" : "+v"(li) :: "memory");
#pragma unroll
  for (int j = 0; j < J; ++j) asm volatile("" : "+v"(o[j][0]), "+v"(o[j][1]) :: "memory");
  if (il >= k || lane >= 4 * J) li = kNegInf;
  float mx = li;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
  const float nt = fmaxf(top, mx);   // finite once any piece has a token
  const float sc = nt == kNegInf ? 0.f : __builtin_amdgcn_exp2f(top - nt);
  const float w = li == kNegInf ? 0.f : __builtin_amdgcn_exp2f(li - nt);
  float ws = w;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) ws += __shfl_xor(ws, sh);
  den = den * sc + ws;
  acc[0] *= sc;
  acc[1] *= sc;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const float wi = __shfl(w, 4 * j + p);
    acc[0] += wi * o[j][0];
    acc[1] += wi * o[j][1];
  }
  top = nt;
}

// part_o and part_lse are not marked __restrict__: loads from restrict
// read-only arguments may be re-issued next to their uses to save registers,
// which would serialise the round's loads.
// Merge records of up to kArgMerges split sequences travel in the kernel
// arguments: a workgroup reads its record together with the other arguments
// instead of one memory round trip later.
constexpr int kArgMerges = 256;
struct MergeRecords {
  int32_t v[3 * kArgMerges];   // (b, first_slot, n_segments) per record
};

// One single-wave workgroup per (merge record, query head): a long record's
// loads spread over as many CUs as it has heads.
template <bool kInArgs>
__global__ __launch_bounds__(64) void merge_kernel(const int32_t* __restrict__ merges,
                                                    const MergeRecords recs,
                                                    const float* part_o, const float* part_lse,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse) {
  int b, first, k;
  if (kInArgs) {
    b = recs.v[3 * blockIdx.x];
    first = recs.v[3 * blockIdx.x + 1];
    k = recs.v[3 * blockIdx.x + 2];
  } else {
    const int32_t* m = merges + 4 * blockIdx.x;
    b = m[0];
    first = m[1];
    k = m[2];
  }
  const int lane = threadIdx.x;
  const int h = blockIdx.y;
  float top = kNegInf, den = 0.f;
  f32x4 acc[2] = {};
  if (k <= 16) {
    if (k > 0) merge_round<4>(part_o, part_lse, first, k, 0, h, lane, top, den, acc);
  } else {
    for (int i0 = 0; i0 < k; i0 += 64)
      merge_round<16>(part_o, part_lse, first, k, i0, h, lane, top, den, acc);
  }
  // Sum the four lane groups (lanes e, e + 16, e + 32, e + 48).
#pragma unroll
  for (int x = 0; x < 2; ++x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[x][i];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[x][i] = v;
    }
  }
  if (lane < 16) {
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    const f32x4 a = acc[0] * inv;
    const f32x4 c = acc[1] * inv;
    const u32x4 w = {static_cast<uint32_t>(bf16_bits(a[0])) | (static_cast<uint32_t>(bf16_bits(a[1])) << 16),
                     static_cast<uint32_t>(bf16_bits(a[2])) | (static_cast<uint32_t>(bf16_bits(a[3])) << 16),
                     static_cast<uint32_t>(bf16_bits(c[0])) | (static_cast<uint32_t>(bf16_bits(c[1])) << 16),
                     static_cast<uint32_t>(bf16_bits(c[2])) | (static_cast<uint32_t>(bf16_bits(c[3])) << 16)};
    *reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(b) * kHq + h) * kHeadDim + 8 * lane) = w;
    if (lane == 0) lse[b * kHq + h] = den > 0.f ? top + __log2f(den) : kNegInf;
  }
}

// Records of at most kSmallMerge pieces (the common case: a sequence cut a few
// ways) take a cheaper shape: one single-wave workgroup per (record, four
// heads); lane (hq, e) = (lane / 16, lane % 16) merges dims [8e, 8e + 8) of
// head 4 blockIdx.y + hq over all pieces, so a wave needs nothing from other
// lanes and the launch has a quarter of the waves of one per head (the
// merge's time grows with the number of waves dispatched). All loads are
// issued before any is used.
constexpr int kSmallMerge = 8;

template <bool kInArgs>
__global__ __launch_bounds__(64) void merge_small_kernel(const int32_t* __restrict__ merges,
                                                          const MergeRecords recs,
                                                          const float* part_o,
                                                          const float* part_lse,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  int b, first, k;
  if (kInArgs) {
    b = recs.v[3 * blockIdx.x];
    first = recs.v[3 * blockIdx.x + 1];
    k = recs.v[3 * blockIdx.x + 2];
  } else {
    const int32_t* m = merges + 4 * blockIdx.x;
    b = m[0];
    first = m[1];
    k = m[2];
  }
  const int lane = threadIdx.x;
  const int h = 4 * blockIdx.y + (lane >> 4);
  const int e = lane & 15;
  float top = kNegInf, den = 0.f;
  f32x4 acc[2] = {};
  if (k > 0) {
    float li[kSmallMerge];
    f32x4 o[kSmallMerge][2];
#pragma unroll
    for (int j = 0; j < kSmallMerge; ++j) {
      const int i = first + min(j, k - 1);   // past the end: the last piece again, weight 0
      li[j] = part_lse[static_cast<int64_t>(i) * kHq + h];
      const float* src = part_o + (static_cast<int64_t>(i) * kHq + h) * kHeadDim + 8 * e;
      o[j][0] = *reinterpret_cast<const f32x4*>(src);
      o[j][1] = *reinterpret_cast<const f32x4*>(src + 4);
    }
    // Every load above is issued before any of these statements (they
    // clobber memory), and every use comes after its value passes one.
#pragma unroll
    for (int j = 0; j < kSmallMerge; ++j) asm volatile("" : "+v"(li[j]) :: "memory");
#pragma unroll
    for (int j = 0; j < kSmallMerge; ++j) asm volatile("" : "+v"(o[j][0]), "+v"(o[j][1]) :: "memory");
#pragma unroll
    for (int j = 0; j < kSmallMerge; ++j)
      if (j < k) top = fmaxf(top, li[j]);
    if (top != kNegInf) {
#pragma unroll
      for (int j = 0; j < kSmallMerge; ++j) {
        const float wj = (j < k && li[j] != kNegInf) ? __builtin_amdgcn_exp2f(li[j] - top) : 0.f;
        den += wj;
        acc[0] += wj * o[j][0];
        acc[1] += wj * o[j][1];
      }
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const f32x4 a = acc[0] * inv;
  const f32x4 c = acc[1] * inv;
  const u32x4 wd = {static_cast<uint32_t>(bf16_bits(a[0])) | (static_cast<uint32_t>(bf16_bits(a[1])) << 16),
                    static_cast<uint32_t>(bf16_bits(a[2])) | (static_cast<uint32_t>(bf16_bits(a[3])) << 16),
                    static_cast<uint32_t>(bf16_bits(c[0])) | (static_cast<uint32_t>(bf16_bits(c[1])) << 16),
                    static_cast<uint32_t>(bf16_bits(c[2])) | (static_cast<uint32_t>(bf16_bits(c[3])) << 16)};
  *reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(b) * kHq + h) * kHeadDim + 8 * e) = wd;
  if (e == 0) lse[b * kHq + h] = den > 0.f ? top + __log2f(den) : kNegInf;
}

}  // namespace

hipError_t launch_decode_partial(const int32_t* workers, const int32_t* segments,
                                 const FirstSegments& firsts, int32_t n_workers,
                                 const uint16_t* q, const uint16_t* k_pool,
                                 const uint16_t* v_pool, const KvAddressing& addr,
                                 float sm_scale_log2, uint16_t* out, float* lse, float* part_o,
                                 float* part_lse, DecodeEngine engine, hipEvent_t start_event,
                                 hipEvent_t stop_event, hipStream_t stream) {
  if (n_workers <= 0) return hipSuccess;
  const bool table = addr.kv_indptr == nullptr;
  auto kernel = engine == DecodeEngine::kDot2
                    ? (table ? decode_partial_kernel<true, Dot2Engine>
                             : decode_partial_kernel<false, Dot2Engine>)
                    : (table ? decode_partial_kernel<true, MfmaEngine>
                             : decode_partial_kernel<false, MfmaEngine>);
  if (start_event != nullptr) {
    // The events take the kernel's own start and end times.
    hipExtLaunchKernelGGL(kernel, dim3(n_workers), dim3(kThreads), 0, stream, start_event,
                          stop_event, 0, workers, segments, firsts, q, k_pool, v_pool, addr,
                          sm_scale_log2, out, lse, part_o, part_lse);
  } else {
    hipLaunchKernelGGL(kernel, dim3(n_workers), dim3(kThreads), 0, stream, workers, segments,
                       firsts, q, k_pool, v_pool, addr, sm_scale_log2, out, lse, part_o, part_lse);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const int32_t* merges, const int32_t* merges_host, int32_t n_merges,
                        int32_t max_pieces, const float* part_o, const float* part_lse,
                        uint16_t* out, float* lse, hipStream_t stream) {
  if (n_merges <= 0) return hipSuccess;
  MergeRecords recs{};
  const bool in_args = merges_host != nullptr && n_merges <= kArgMerges;
  if (in_args) {
    for (int i = 0; i < n_merges; ++i) {
      recs.v[3 * i] = merges_host[4 * i];
      recs.v[3 * i + 1] = merges_host[4 * i + 1];
      recs.v[3 * i + 2] = merges_host[4 * i + 2];
    }
  }
  if (max_pieces <= kSmallMerge) {
    if (in_args)
      hipLaunchKernelGGL(merge_small_kernel<true>, dim3(n_merges, kHq / 4), dim3(64), 0, stream,
                         merges, recs, part_o, part_lse, out, lse);
    else
      hipLaunchKernelGGL(merge_small_kernel<false>, dim3(n_merges, kHq / 4), dim3(64), 0, stream,
                         merges, recs, part_o, part_lse, out, lse);
  } else if (in_args) {
    hipLaunchKernelGGL(merge_kernel<true>, dim3(n_merges, kHq), dim3(64), 0, stream, merges, recs,
                       part_o, part_lse, out, lse);
  } else {
    hipLaunchKernelGGL(merge_kernel<false>, dim3(n_merges, kHq), dim3(64), 0, stream, merges, recs,
                       part_o, part_lse, out, lse);
  }
  return hipGetLastError();
}

}  // namespace pkv
