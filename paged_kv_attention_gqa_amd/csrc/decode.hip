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
// * Both contractions run on v_mfma_f32_16x16x32_bf16, the 8 query heads
//   padded to 16 MFMA columns:
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
// * Loads are software-pipelined one tile ahead (page ids two tiles ahead);
//   out-of-range tokens of the last tile re-read the item's last page, which
//   keeps every load unconditional, and get score -inf, i.e. weight exactly 0.
// * Scores are scaled by sm_scale*log2(e) in fp32 and exponentiated with
//   exp2; the running max is reduced across the 4 lane rows with the
//   cross-lane swaps v_permlane16_swap / v_permlane32_swap (vector ALU, no
//   LDS), the running sum is kept per lane and reduced once at the end.
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

constexpr int kGroup = kHq / kHkv;      // query heads per KV head
constexpr int kTileTok = 32;            // tokens per wave per step
constexpr int kRowU16 = kHeadDim + 16;  // LDS row of one token's V: 256 B + 32 B pad
constexpr int kWaveLdsU16 = kTileTok * kRowU16;
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

__device__ __forceinline__ void compute_tile(const Tile& t, int t0, int n, const u32x4 (&qf)[4],
                                             float scale_log2, int r, int c, uint16_t* lw,
                                             Softmax& st) {
  // Scores of the 32 tokens against the (padded) 16 heads.
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

  bf16x8 pb;
#pragma unroll
  for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(p[j]);

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
template <bool kTable>
__device__ __forceinline__ void process_segment(
    const TokenRows<kTable>& ids, int b, int n, int slot, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, uint16_t* lds) {
  const int lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // KV head of this wave
  const int r = lane & 15;
  const int c = lane >> 4;
  const int head = g * kGroup + r;   // a real query head only for r < kGroup
  const int last = n - 1;

  // The ids of the first two tiles are fetched first: they depend only on
  // the segment's position, so (for a worker's first segment, whose position
  // comes with the kernel arguments) they leave before q, which needs b.
  const int ja0 = min(r, last), ja1 = min(16 + r, last);
  const int jn0 = min(kTileTok + r, last), jn1 = min(kTileTok + 16 + r, last);
  int32_t a0 = ids.fetch(ja0), a1 = ids.fetch(ja1);
  int32_t n0 = ids.fetch(jn0), n1 = ids.fetch(jn1);

  // Q as the B operand: lane (r, c) holds q[head r][32x + 8c, +8) for k-step x.
  // The 8 padding columns (r >= kGroup) repeat heads r - kGroup: their scores
  // and outputs are computed and never stored, and every lane loads, so the
  // compiler can count the loads in flight (a masked load made it wait for q
  // before the first K/V loads).
  u32x4 qf[4];
  {
    const uint16_t* qh =
        q + (static_cast<int64_t>(b) * kHq + g * kGroup + (r & (kGroup - 1))) * kHeadDim + 8 * c;
#pragma unroll
    for (int x = 0; x < 4; ++x) qf[x] = *reinterpret_cast<const u32x4*>(qh + 32 * x);
  }

  Softmax st;
#pragma unroll
  for (int db = 0; db < 8; ++db) st.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.l = 0.f;
  uint16_t* lw = lds + g * kWaveLdsU16;   // each wave owns its LDS slice

  // Software pipeline over a ring of kPipeTiles register buffers: while the
  // oldest tile is computed, the next kPipeTiles - 1 tiles are in flight.
  // Page ids are fetched one tile ahead of the K/V loads they feed and issued
  // before them, so waiting for ids never waits for younger K/V loads. The
  // loop is unrolled over the ring so every buffer index is a constant, its
  // body has no early exit, and the empty asm statements keep each load group
  // where it is written. Loads past the segment re-read its last row; the
  // last n_tiles % kPipeTiles tiles are computed after the loop from the
  // buffers the final iterations loaded.
  const int n_tiles = (n + kTileTok - 1) / kTileTok;
  const int n_rounds = n_tiles / kPipeTiles;
  static_assert(kPipeTiles == 2, "the prologue below fills a ring of two tiles");
  Tile ring[kPipeTiles];
  // The first two tiles' ids (fetched above) are all in before any K/V load,
  // so the loop starts with the second tile's rows known and no load pending
  // but the first tile's.
  asm volatile("" : "+v"(a0), "+v"(a1), "+v"(n0), "+v"(n1));
  load_tile(ring[0], k_pool, v_pool, ids.row_of(a0, ja0), ids.row_of(a1, ja1), g, c);
  int32_t next0 = ids.row_of(n0, jn0);
  int32_t next1 = ids.row_of(n1, jn1);
  int t0 = 0;
  for (int round = 0; round < n_rounds; ++round) {
#pragma unroll
    for (int k = 0; k < kPipeTiles; ++k) {
      // compute tile round * kPipeTiles + k (ring[k]); load the tile
      // kPipeTiles - 1 later into the buffer computed last; fetch the ids of
      // the tile after that.
      asm volatile("" ::: "memory");
      const int tf = t0 + kTileTok * (k + kPipeTiles);
      const int j0 = min(tf + r, last);
      const int j1 = min(tf + 16 + r, last);
      int32_t f0 = ids.fetch(j0);
      int32_t f1 = ids.fetch(j1);
      load_tile(ring[(k + kPipeTiles - 1) % kPipeTiles], k_pool, v_pool, next0, next1, g, c);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      compute_tile(ring[k], t0 + kTileTok * k, n, qf, scale_log2, r, c, lw, st);
      __builtin_amdgcn_sched_barrier(0);
      // The fetched ids stay opaque until the compute above has been issued,
      // so nothing derived from them is scheduled next to their loads (which
      // would make the wave wait for loads it has just issued).
      asm volatile("" : "+v"(f0), "+v"(f1));
      next0 = ids.row_of(f0, j0);
      next1 = ids.row_of(f1, j1);
    }
    t0 += kTileTok * kPipeTiles;
  }
  const int rest = n_tiles - n_rounds * kPipeTiles;
#pragma unroll
  for (int k = 0; k < kPipeTiles - 1; ++k)
    if (k < rest) compute_tile(ring[k], t0 + kTileTok * k, n, qf, scale_log2, r, c, lw, st);

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

// One workgroup per worker: it walks its segments in order. The first
// kFirstArgWorkers workers find where their first segment's ids start in the
// kernel arguments (CSR: (kv_indptr[b] + tok_begin, 0, n); block table: (b,
// tok_begin, n); n = 0 if the worker has no segment), so its id loads leave
// one memory round trip earlier than the worker's record, which still
// supplies b, the slot and the segment range.
template <bool kTable>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_partial_kernel(
    const int32_t* __restrict__ workers, const int32_t* __restrict__ segments,
    const FirstSegments firsts, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool, KvAddressing addr,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[kHkv * kWaveLdsU16];
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
      process_segment<kTable>(ids, wrec[0], n, wrec[3], q, k_pool, v_pool, scale_log2, out, lse,
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
      process_segment<kTable>(ids, seg[0], n, seg[3], q, k_pool, v_pool, scale_log2, out, lse,
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
                                 float* part_lse, hipStream_t stream) {
  if (n_workers <= 0) return hipSuccess;
  if (addr.kv_indptr == nullptr) {
    hipLaunchKernelGGL(decode_partial_kernel<true>, dim3(n_workers), dim3(kThreads), 0, stream,
                       workers, segments, firsts, q, k_pool, v_pool, addr,
                       sm_scale_log2, out, lse, part_o, part_lse);
  } else {
    hipLaunchKernelGGL(decode_partial_kernel<false>, dim3(n_workers), dim3(kThreads), 0, stream,
                       workers, segments, firsts, q, k_pool, v_pool, addr,
                       sm_scale_log2, out, lse, part_o, part_lse);
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
