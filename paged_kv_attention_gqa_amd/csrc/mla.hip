// Index-gather latent-attention decode for gfx950 (MI355X), over a bf16 pool
// or a pool of 656-byte FP8 tokens.
//
// What is computed follows the FlagGems flash_mla_with_kvcache page
// (_sparse_decode_kernel, bf16 mode): for row b every list entry
// t = indices[b, i] with 0 <= t < pool_tokens selects pool row kv[t]
// (576 bf16: scores use all 576 dims, values are the first 512 dims); other
// entries are masked. Scores are scaled by sm_scale, reduced with an online
// softmax, and the output is bf16 with a base-2 LSE.
//
// Design:
// * Work is split three ways: row b, a block of up to 64 query heads, and a
//   contiguous piece of the index list; one workgroup of 8 waves per triple.
//   The two head blocks of one (row, piece) are launched 8 workgroups apart,
//   so they run on the same XCD and the second gather of a tile mostly hits
//   in that XCD's L2 (without this the memory-side fetches were twice the
//   gathered bytes).
//   Wave w owns 16 heads (w % 4) and one half (w / 4) of both contractions:
//   dims [288 half, +288) of the 576-dim scores and dims [256 half, +256) of
//   the 512-dim output. The two waves of a head group swap their partial
//   scores through LDS, so both hold the full scores, run the same softmax,
//   and each accumulates its half of the output: no MFMA work is repeated and
//   each wave keeps 36 registers of Q and 64 of accumulators, which lets two
//   waves share each SIMD. Pieces of one (row, head block) leave normalised
//   fp32 partials that a second kernel merges by LSE (vLLM fork qsa.py,
//   _qsa_merge_splitk_kernel); with a single piece the output is final.
// * 128 heads share every gathered row, so both contractions are dense and
//   run on v_mfma_f32_16x16x32_bf16:
//     S^T[tok, h] = K[tok, :] . Q[h, :]        A = K rows from LDS, B = Q^T (registers)
//     O^T[d, h]  += V^T[d, tok] . P^T[tok, h]  A = V^T read with ds_read_b64_tr_b16
//   The transposing LDS read hands each lane four tokens of one dim, so V is
//   never rewritten transposed. The S^T accumulator already holds each lane's
//   P^T operand (head = lane % 16, tokens 16h + 4c + j), as in the GQA kernel.
// * A tile is 32 gathered rows (36 KB): sixteen threads per row load it with
//   16-byte loads (consecutive lanes on consecutive bytes) into registers two
//   tiles ahead of the compute, then store it to one of three LDS buffers
//   whose rows are padded to 1184 bytes (the padding measured fastest among
//   1168-1280 bytes). One barrier per tile: in the step that finishes tile t
//   (softmax and P.V) each wave also computes its half scores of tile t+1,
//   whose MFMAs overlap the softmax, and the workgroup stores tile t+2.
// * The running max that the exponentials are taken against moves only when
//   a head's max grows by more than 8 (log2 units), so the accumulators are
//   rescaled on few tiles; p stays below 2^8, well inside fp32 and bf16.
// * A masked entry is neither loaded nor stored: its score is -inf (weight 0)
//   and its LDS row keeps older finite data (the buffers start zeroed). A
//   piece with no valid entry gives out 0 and lse -inf.
// * Optional per-row list lengths (HAVE_TOPK_LENGTH on the page) shorten each
//   piece to the entries before min(max(len, 0), topk). An optional sink logit
//   per head (HAVE_ATTN_SINK) joins the softmax denominator with no value:
//   the finished output is sum_j e^s_j v_j / (sum_j e^s_j + e^sink), applied
//   where the output is finished (here for one piece, else in the merge), and
//   the LSE stays that of the entries alone, as the page stores it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lanes.h"
#include "mla.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileTok = 32;
constexpr int kUnitsPerRow = kMlaDqk / 8;          // 72 units of 16 bytes
constexpr int kRowU16 = kMlaDqk + 16;              // LDS row: 1152 B + 32 B pad
constexpr int kBufU16 = kTileTok * kRowU16;        // one tile buffer
constexpr int kThreads = 512;                      // 8 waves
constexpr int kHeadsPerWave = 16;
constexpr int kHeadBlock = 4 * kHeadsPerWave;      // 64 heads per workgroup
constexpr int kQSteps = kMlaDqk / 32 / 2;          // 9 k-steps of 32 dims per half
constexpr int kVBlocks = kMlaDv / 16 / 2;          // 16 blocks of 16 dims per half
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats rounded to bf16 (nearest, ties to even), first in the low half.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return static_cast<uint32_t>(bf16_bits(a)) | (static_cast<uint32_t>(bf16_bits(b)) << 16);
}

// Thread t stages tile row t / 16: 16-byte units (t % 16) + 16 u, u = 0..4
// (the last only for t % 16 < 8), so sixteen consecutive lanes read 256
// contiguous bytes of one row and every thread needs one list entry per tile.
constexpr int kThreadsPerRow = kThreads / kTileTok;   // 16
constexpr int kLoadsPerThread = (kUnitsPerRow + kThreadsPerRow - 1) / kThreadsPerRow;   // 5

// Row staging of the bf16 pool (576 bf16 = 72 units of 16 bytes per row).
struct StagedBf16 {
  u32x4 v[kLoadsPerThread];
  bool valid;

  __device__ __forceinline__ static bool has_unit(int u) {
    return u * kThreadsPerRow + static_cast<int>(threadIdx.x % kThreadsPerRow) < kUnitsPerRow;
  }

  // Every load is issued, so the compiler can count the loads in flight: a
  // masked entry reads the in-bounds row `safe` instead (never stored, so
  // never used), and the fifth unit of threads past the row's end re-reads
  // the row's last unit.
  __device__ __forceinline__ void load(int32_t id, int64_t pool_tokens, const void* kv,
                                       const void* safe) {
    valid = id >= 0 && static_cast<int64_t>(id) < pool_tokens;
    const uint16_t* row = valid ? static_cast<const uint16_t*>(kv) + static_cast<int64_t>(id) * kMlaDqk
                                : static_cast<const uint16_t*>(safe);
    const int j = static_cast<int>(threadIdx.x % kThreadsPerRow);
#pragma unroll
    for (int u = 0; u < kLoadsPerThread; ++u)
      v[u] = *reinterpret_cast<const u32x4*>(row + min(j + u * kThreadsPerRow, kUnitsPerRow - 1) * 8);
  }

  // A masked row is not stored; only its flag is cleared.
  __device__ __forceinline__ void store(uint16_t* buf, uint8_t* vflag) const {
    const int row = threadIdx.x / kThreadsPerRow;
    uint16_t* dst = buf + row * kRowU16 + (threadIdx.x % kThreadsPerRow) * 8;
    if (threadIdx.x % kThreadsPerRow == 0) vflag[row] = valid ? 1 : 0;
    if (!valid) return;
#pragma unroll
    for (int u = 0; u < kLoadsPerThread; ++u)
      if (has_unit(u)) *reinterpret_cast<u32x4*>(dst + u * kThreadsPerRow * 8) = v[u];
  }
};

// Row staging of the FP8 pool: 656-byte tokens, e4m3 values [0, 512), four
// fp32 scales [512, 528) (scale k for values 128k .. 128k+127), 64 bf16 values
// [528, 656). Thread j of a row loads the e4m3 units j and j + 16 (values
// 16j and 256 + 16j, +16), the scale unit, and for j < 8 the bf16 unit j; at
// the store it multiplies each value by its scale in fp32 and rounds to bf16,
// so the LDS tile has the same 576-bf16 rows as the bf16 pool.
struct StagedFp8 {
  u32x4 codes[2];
  u32x4 scales;
  u32x4 tail;
  bool valid;

  // As for bf16 rows, every load is issued (masked entries read `safe`;
  // threads j >= 8 re-read a tail unit they do not store).
  __device__ __forceinline__ void load(int32_t id, int64_t pool_tokens, const void* kv,
                                       const void* safe) {
    valid = id >= 0 && static_cast<int64_t>(id) < pool_tokens;
    const int j = threadIdx.x % kThreadsPerRow;
    const uint8_t* src = valid ? static_cast<const uint8_t*>(kv) + static_cast<int64_t>(id) * kMlaFp8TokenBytes
                               : static_cast<const uint8_t*>(safe);
    codes[0] = *reinterpret_cast<const u32x4*>(src + 16 * j);
    codes[1] = *reinterpret_cast<const u32x4*>(src + 256 + 16 * j);
    scales = *reinterpret_cast<const u32x4*>(src + 512);
    tail = *reinterpret_cast<const u32x4*>(src + 528 + 16 * (j & 7));
  }

  __device__ __forceinline__ void store(uint16_t* buf, uint8_t* vflag) const {
    const int row = threadIdx.x / kThreadsPerRow;
    const int j = threadIdx.x % kThreadsPerRow;
    uint16_t* dst = buf + row * kRowU16;
    if (j == 0) vflag[row] = valid ? 1 : 0;
    if (!valid) return;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // values 256u + 16j .. +16 lie in the 128-value block 2u + j / 8 (the
      // element is copied out first: a bit cast applied directly to a vector
      // element compiled as a cast of element 0)
      const uint32_t sc_bits = j < 8 ? scales[2 * u] : scales[2 * u + 1];
      const float sc = __builtin_bit_cast(float, sc_bits);
      uint32_t packed[8];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const int word = static_cast<int>(codes[u][wd]);
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);   // bytes 0, 1
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);    // bytes 2, 3
        packed[2 * wd] = bf16_pair(lo[0] * sc, lo[1] * sc);
        packed[2 * wd + 1] = bf16_pair(hi[0] * sc, hi[1] * sc);
      }
      const u32x4 a = {packed[0], packed[1], packed[2], packed[3]};
      const u32x4 b = {packed[4], packed[5], packed[6], packed[7]};
      uint16_t* d = dst + 256 * u + 16 * j;
      *reinterpret_cast<u32x4*>(d) = a;
      *reinterpret_cast<u32x4*>(d + 8) = b;
    }
    if (j < 8) *reinterpret_cast<u32x4*>(dst + 512 + 8 * j) = tail;
  }
};

// Entry of this thread's row in the tile starting at t0, as loaded (the load
// is always issued, clamped into the piece; n >= 1), and whether that row
// lies inside the piece. The two are combined only where the entry is used,
// so nothing is computed from the loaded value next to its load (which would
// make the wave wait for the load, and for every load before it, at once).
struct Entry {
  int32_t id;
  bool in_piece;
};
__device__ __forceinline__ Entry tile_entry(const int32_t* __restrict__ idx, int t0, int n) {
  const int tok = t0 + static_cast<int>(threadIdx.x) / kThreadsPerRow;
  return Entry{idx[min(tok, n - 1)], tok < n};
}
__device__ __forceinline__ int32_t entry_id(Entry e) {
  int32_t id = e.id;
  asm volatile("" : "+v"(id));
  return e.in_piece ? id : -1;
}

struct State {
  f32x4 acc[kVBlocks];   // acc[db][i] = O[head r][256 half + 16 db + 4c + i]
  float m;               // running max (log2 domain), equal on the 4 lane rows
  float l;               // this lane's share of the exp-sum
};

// This wave's half of the scores of one tile: S^T over dims [288 half, +288).
__device__ __forceinline__ void half_scores(const uint16_t* buf, const u32x4 (&qf)[kQSteps],
                                            int half, int r, int c, f32x4& s0, f32x4& s1) {
  // Four accumulator chains (rows 0-15 / 16-31, even / odd k-steps) keep
  // consecutive MFMAs from waiting on each other.
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
  const uint16_t* row0 = buf + r * kRowU16 + 8 * c + 288 * half;
  const uint16_t* row1 = row0 + 16 * kRowU16;
#pragma unroll
  for (int ks = 0; ks < kQSteps; ++ks) {
    const u32x4 k0 = *reinterpret_cast<const u32x4*>(row0 + 32 * ks);
    const u32x4 k1 = *reinterpret_cast<const u32x4*>(row1 + 32 * ks);
    if (ks & 1) {
      b0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k0), as_bf16x8(qf[ks]), b0, 0, 0, 0);
      b1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k1), as_bf16x8(qf[ks]), b1, 0, 0, 0);
    } else {
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k0), as_bf16x8(qf[ks]), a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k1), as_bf16x8(qf[ks]), a1, 0, 0, 0);
    }
  }
  s0 = a0 + b0;
  s1 = a1 + b1;
}

// Online-softmax update with the full scores s0/s1 (identical in both waves of
// a head group, since a + b == b + a exactly), then this wave's half of P.V.
__device__ __forceinline__ void softmax_pv(const uint16_t* buf, const uint8_t* vflag, f32x4 s0,
                                           f32x4 s1, float scale_log2, int half, int r, int c,
                                           State& st) {
  // p[4h + j] belongs to tile row 16h + 4c + j.
  float p[8];
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = vflag[4 * c + j] ? s0[j] * scale_log2 : kNegInf;
    p[4 + j] = vflag[16 + 4 * c + j] ? s1[j] * scale_log2 : kNegInf;
    mx = fmaxf(mx, fmaxf(p[j], p[4 + j]));
  }
  mx = max_xor32(max_xor16(mx));
  // The reference max moves only when a head's max grows by more than
  // kRescaleSlack (log2 units), so the accumulators are rarely rescaled;
  // meanwhile p stays below 2^kRescaleSlack.
  const float m_new = fmaxf(st.m, mx);
  const bool grow = m_new > st.m + kRescaleSlack;   // false while both are -inf
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    asm volatile("" ::: "memory");   // keeps this rarely taken block a branch
    const float m_ref = grow ? m_new : st.m;
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m - m_ref) : 1.0f;   // 0 from -inf
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < kVBlocks; ++db) st.acc[db] *= alpha;
    st.m = m_ref;
  }
  const float m_use = (st.m == kNegInf) ? 0.f : st.m;   // no valid entry yet: every p is 0
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __builtin_amdgcn_exp2f(p[j] - m_use);
    psum += p[j];
  }
  st.l += psum;
  bf16x8 pb;
#pragma unroll
  for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(p[j]);

  // V^T operand: lane (r, c) needs dim 256 half + 16 db + r of tile rows
  // 16h + 4c + j. Within each 16-lane group the transposing read gives lane i
  // element i%4 of the 8-byte chunks addressed by lanes 4j + i/4, so lane
  // (r, c) points at row 16h + 4c + r/4, dims 256 half + 16 db + 4 (r%4) .. +4.
  const uint16_t* vrow0 = buf + (4 * c + (r >> 2)) * kRowU16 + 4 * (r & 3) + 256 * half;
  const uint16_t* vrow1 = vrow0 + 16 * kRowU16;
#pragma unroll
  for (int db = 0; db < kVBlocks; ++db) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vrow0 + 16 * db));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vrow1 + 16 * db));
    const u32x4 a = {__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                     __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]};
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), pb, st.acc[db], 0, 0, 0);
  }
}

// grid: (pieces, head blocks, batch). Each workgroup decodes list entries
// [piece * per_piece, +per_piece) of row b for heads [64 hb, 64 hb + 64).
template <typename Staged>
__global__ __launch_bounds__(kThreads) void mla_partial_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv, int64_t pool_tokens,
    const int32_t* __restrict__ indices, int topk, int num_qo_heads, int per_piece, int pieces,
    int hblocks, int batch, float scale_log2, const float* __restrict__ attn_sink,
    const int32_t* __restrict__ topk_length, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * kBufU16];
  __shared__ uint8_t vflag[3][kTileTok];
  __shared__ f32x4 xscore[2][8][2][64];   // half scores by tile parity, [wave][mb][lane]
  // Workgroups are dealt to the XCDs in turn (workgroup i to XCD i % 8). With
  // two head blocks, workgroups 16 g + x and 16 g + 8 + x (x < 8) are the two
  // head blocks of one (row, piece), so they share an XCD and its L2, and the
  // second gather of each tile mostly hits there.
  const int wg = blockIdx.x;
  const int pair = hblocks == 2 ? (wg >> 4) * 8 + (wg & 7) : wg;
  const int hb = hblocks == 2 ? (wg >> 3) & 1 : 0;
  if (pair >= pieces * batch) return;   // padding of the last group of 16
  const int b = pair / pieces;
  const int piece = pair - b * pieces;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hg = w & 3;          // head group
  const int half = w >> 2;       // which half of both contractions
  const int partner = w ^ 4;
  const int r = lane & 15;
  const int c = lane >> 4;
  const int head = hb * kHeadBlock + hg * kHeadsPerWave + r;
  const bool head_ok = head < num_qo_heads;
  const bool group_ok = hb * kHeadBlock + hg * kHeadsPerWave < num_qo_heads;
  const int t_begin = piece * per_piece;
  const int row_len = topk_length != nullptr ? min(max(topk_length[b], 0), topk) : topk;
  const int n = min(per_piece, row_len - t_begin);   // entries of this piece (may be <= 0)
  const int32_t* idx = indices + static_cast<int64_t>(b) * topk + t_begin;

  u32x4 qf[kQSteps];
  {
    const uint16_t* qh = q + (static_cast<int64_t>(b) * num_qo_heads + (head_ok ? head : 0)) * kMlaDqk +
                         288 * half + 8 * c;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks)
      qf[ks] = head_ok ? *reinterpret_cast<const u32x4*>(qh + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
  }
  State st;
#pragma unroll
  for (int db = 0; db < kVBlocks; ++db) st.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.l = 0.f;

  // Pipeline over three LDS tile buffers with one barrier per tile: in step t
  // the workgroup stores tile t+2 (loaded two steps earlier into one of two
  // register sets) and reloads that set with tile t+4, finishes tile t
  // (partner's half scores, softmax, P.V) and computes its half scores of
  // tile t+1. Entries past the piece read as -1 (masked, nothing loaded).
  const int n_tiles = n > 0 ? (n + kTileTok - 1) / kTileTok : 0;
  // An in-bounds row for the loads of masked entries: pool row 0, or this
  // row's q (at least one 1152-byte row) when the pool is empty.
  const void* safe = pool_tokens > 0 ? kv : static_cast<const void*>(q + static_cast<int64_t>(b) * num_qo_heads * kMlaDqk);
  Staged sa, sb;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
  if (n_tiles > 0) {
    // A masked row is neither loaded nor stored, so its slot keeps older data:
    // zeros from here, or a row staged for an earlier tile. Either is finite
    // unless the pool itself holds a non-finite value in a row that was used.
    {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      for (int i = threadIdx.x; i < 3 * kBufU16 / 8; i += kThreads)
        reinterpret_cast<u32x4*>(lds)[i] = zero;
    }
    sa.load(entry_id(tile_entry(idx, 0, n)), pool_tokens, kv, safe);
    sb.load(entry_id(tile_entry(idx, kTileTok, n)), pool_tokens, kv, safe);
    __syncthreads();   // every wave's zeros land before any wave stores a row
    Entry id_a = tile_entry(idx, 2 * kTileTok, n);
    Entry id_b = tile_entry(idx, 3 * kTileTok, n);
    // Loads leave in the loop's order (a set's rows, then the entry it loads
    // next), so the loop starts with the same loads pending as every step.
    sa.store(lds, vflag[0]);
    sa.load(entry_id(id_a), pool_tokens, kv, safe); // tile 2
    id_a = tile_entry(idx, 4 * kTileTok, n);
    sb.store(lds + kBufU16, vflag[1]);
    sb.load(entry_id(id_b), pool_tokens, kv, safe); // tile 3
    id_b = tile_entry(idx, 5 * kTileTok, n);
    __syncthreads();
    if (group_ok) {
      half_scores(lds, qf, half, r, c, s0, s1);
      xscore[0][w][0][lane] = s0;
      xscore[0][w][1][lane] = s1;
    }
    __syncthreads();
    int cur = 0;                                    // buffer of tile t
    // Step tt: store tile tt+2 from `set`, reload `set` with tile tt+4, fetch
    // the entry of tile tt+6, then finish tile tt and score tile tt+1.
    auto step = [&](int tt, Staged& set, Entry& id_set) {
      const int nxt = cur == 2 ? 0 : cur + 1;       // buffer of tile tt+1
      const int far = nxt == 2 ? 0 : nxt + 1;       // buffer of tile tt+2
      set.store(lds + far * kBufU16, vflag[far]);   // tile tt+2
      set.load(entry_id(id_set), pool_tokens, kv, safe);   // tile tt+4
      id_set = tile_entry(idx, (tt + 6) * kTileTok, n);
      if (group_ok) {
        const f32x4 f0 = s0 + xscore[tt & 1][partner][0][lane];
        const f32x4 f1 = s1 + xscore[tt & 1][partner][1][lane];
        // Scores of tile tt+1 first (in the last step they are computed from
        // a buffer holding finite older data and never used): their MFMAs
        // run while the softmax of tile tt is on the vector ALU.
        half_scores(lds + nxt * kBufU16, qf, half, r, c, s0, s1);
        softmax_pv(lds + cur * kBufU16, vflag[cur], f0, f1, scale_log2, half, r, c, st);
        xscore[(tt + 1) & 1][w][0][lane] = s0;
        xscore[(tt + 1) & 1][w][1][lane] = s1;
      }
      __syncthreads();
      cur = nxt;
    };
    // Whole pairs of steps in the loop and an odd last step after it, so the
    // loop never leaves between the two steps of a pair (which would give the
    // loop head a path with fewer loads in flight, and the compiler would
    // then wait for every load at the top of each pair).
    int t = 0;
    for (; t + 1 < n_tiles; t += 2) {
      step(t, sa, id_a);
      step(t + 1, sb, id_b);
    }
    if (t < n_tiles) step(t, sa, id_a);
  }

  const float l_tot = sum_xor32(sum_xor16(st.l));
  const bool any = l_tot > 0.f;
  const float lse2 = any ? st.m + __log2f(l_tot) : kNegInf;
  if (!head_ok) return;
  if (pieces == 1) {
    // sum_j 2^(t_j) = l_tot * 2^m in the log2 domain; the sink adds 2^(sink * log2 e).
    const float sink_rel = (attn_sink != nullptr && any)
                               ? __builtin_amdgcn_exp2f(attn_sink[head] * kLog2e - st.m)
                               : 0.f;
    const float inv = any ? 1.0f / (l_tot + sink_rel) : 0.f;
    uint16_t* o = out + (static_cast<int64_t>(b) * num_qo_heads + head) * kMlaDv + 256 * half + 4 * c;
#pragma unroll
    for (int db = 0; db < kVBlocks; ++db) {
      const f32x4 v = st.acc[db] * inv;
      const u32x2 wds = {static_cast<uint32_t>(bf16_bits(v[0])) | (static_cast<uint32_t>(bf16_bits(v[1])) << 16),
                         static_cast<uint32_t>(bf16_bits(v[2])) | (static_cast<uint32_t>(bf16_bits(v[3])) << 16)};
      *reinterpret_cast<u32x2*>(o + 16 * db) = wds;
    }
    if (c == 0 && half == 0) lse[static_cast<int64_t>(b) * num_qo_heads + head] = lse2;
  } else {
    const float inv = any ? 1.0f / l_tot : 0.f;
    const int64_t slot = (static_cast<int64_t>(b) * num_qo_heads + head) * pieces + piece;
    float* o = part_o + slot * kMlaDv + 256 * half + 4 * c;
#pragma unroll
    for (int db = 0; db < kVBlocks; ++db) *reinterpret_cast<f32x4*>(o + 16 * db) = st.acc[db] * inv;
    if (c == 0 && half == 0) part_lse[slot] = lse2;
  }
}

// One 128-thread workgroup per (row, head): thread t owns dims 4t .. 4t+3 and
// folds the pieces in order.
__global__ __launch_bounds__(128) void mla_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        int pieces, int num_qo_heads,
                                                        const float* __restrict__ attn_sink,
                                                        uint16_t* __restrict__ out,
                                                        float* __restrict__ lse) {
  const int64_t bh = blockIdx.x;
  const float* pl = part_lse + bh * pieces;
  float top = kNegInf;
  for (int i = 0; i < pieces; ++i) top = fmaxf(top, pl[i]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (top != kNegInf) {
    for (int i = 0; i < pieces; ++i) {
      const float li = pl[i];
      const float wgt = (li == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(li - top);
      den += wgt;
      acc += wgt * *reinterpret_cast<const f32x4*>(part_o + (bh * pieces + i) * kMlaDv + 4 * threadIdx.x);
    }
  }
  // With a sink: sum_i 2^(lse_i) o_i / (sum_i 2^(lse_i) + 2^(sink log2 e)), all scaled by 2^-top.
  const float sink_rel = (attn_sink != nullptr && den > 0.f)
                             ? __builtin_amdgcn_exp2f(attn_sink[bh % num_qo_heads] * kLog2e - top)
                             : 0.f;
  const float inv = den > 0.f ? 1.0f / (den + sink_rel) : 0.f;
  const u32x2 wds = {static_cast<uint32_t>(bf16_bits(acc[0] * inv)) | (static_cast<uint32_t>(bf16_bits(acc[1] * inv)) << 16),
                     static_cast<uint32_t>(bf16_bits(acc[2] * inv)) | (static_cast<uint32_t>(bf16_bits(acc[3] * inv)) << 16)};
  *reinterpret_cast<u32x2*>(out + bh * kMlaDv + 4 * threadIdx.x) = wds;
  if (threadIdx.x == 0) lse[bh] = den > 0.f ? top + __log2f(den) : kNegInf;
}

// Pieces per (row, head block): enough workgroups to give each CU one, with
// at least two tiles per piece.
int mla_pieces(int32_t batch, int32_t num_qo_heads, int32_t topk, int num_cus) {
  const int hblocks = (num_qo_heads + kHeadBlock - 1) / kHeadBlock;
  const int base = max(1, batch * hblocks);
  int pieces = max(1, (num_cus + base - 1) / base);
  const int max_pieces = max(1, topk / (2 * kTileTok));
  return min(pieces, max_pieces);
}

// The fp32 partials of pkv_gather_mla_noalloc. In host code this name only
// stands for the array: kernels get its device address from mla_scratch.
static __device__ __align__(256) unsigned char scratch[kMlaScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t mla_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int mla_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t d_qk, int32_t d_v,
                        int32_t topk, size_t* bytes, std::string* err) {
  if (batch < 0 || topk < 0) { *err = "batch and topk must be >= 0"; return 1; }
  if (d_qk != kMlaDqk || d_v != kMlaDv) {
    *err = "expected d_qk=576 and d_v=512";
    return 2;
  }
  if (num_qo_heads <= 0 || num_qo_heads % 16 != 0 || num_qo_heads > kMlaMaxHeads) {
    *err = "num_qo_heads must be a multiple of 16 in [16, 128]";
    return 2;
  }
  const int pieces = mla_pieces(batch, num_qo_heads, topk, kMlaPlanCus);
  *bytes = pieces > 1 ? static_cast<size_t>(batch) * num_qo_heads * pieces * (kMlaDv + 1) * sizeof(float) : 0;
  return 0;
}

hipError_t launch_gather_mla(const uint16_t* q, const void* kv_pool, bool fp8_pool,
                             int64_t pool_tokens, const int32_t* indices, int32_t topk,
                             int32_t batch, int32_t num_qo_heads, float sm_scale,
                             const float* attn_sink, const int32_t* topk_length, void* workspace,
                             uint16_t* out, float* lse, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const int pieces = mla_pieces(batch, num_qo_heads, topk, kMlaPlanCus);
  const int per_piece = topk > 0 ? ((topk + pieces - 1) / pieces + kTileTok - 1) / kTileTok * kTileTok : 0;
  const int hblocks = (num_qo_heads + kHeadBlock - 1) / kHeadBlock;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = pieces > 1 ? part_o + static_cast<size_t>(batch) * num_qo_heads * pieces * kMlaDv : nullptr;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  const int pairs = pieces * batch;
  const int grid = hblocks == 2 ? 16 * ((pairs + 7) / 8) : pairs;
  if (fp8_pool) {
    hipLaunchKernelGGL(mla_partial_kernel<StagedFp8>, dim3(grid), dim3(kThreads), 0, stream, q,
                       kv_pool, pool_tokens, indices, topk, num_qo_heads, per_piece, pieces,
                       hblocks, batch, scale_log2, attn_sink, topk_length, out, lse, part_o,
                       part_lse);
  } else {
    hipLaunchKernelGGL(mla_partial_kernel<StagedBf16>, dim3(grid), dim3(kThreads), 0, stream, q,
                       kv_pool, pool_tokens, indices, topk, num_qo_heads, per_piece, pieces,
                       hblocks, batch, scale_log2, attn_sink, topk_length, out, lse, part_o,
                       part_lse);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pieces == 1) return e;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(batch * num_qo_heads), dim3(kMlaDv / 4), 0, stream,
                     part_o, part_lse, pieces, num_qo_heads, attn_sink, out, lse);
  return hipGetLastError();
}

}  // namespace pkv
