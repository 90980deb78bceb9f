// MLA (multi-head latent attention) decode over a paged latent cache.
//
// What is computed (page "字节跳动 AI Infra (2)", question on KV-cache
// principles, the MLA paragraph): the cache holds one latent row c_t per
// token (512 wide); head h's key and value are recovered as
// K_t = c_t W_uk[:, h] and V_t = c_t W_uv[:, h] (head h = column block h of
// the d_c x (H * head_dim) up-projections), and attention then runs as over
// full-width K/V:  out[b][h] = sum_t softmax_t(scale * q[b][h] . K_t) V_t.
//
// The kernels never materialise K or V.  By associativity
//     q . (c_t W_uk_h) = (W_uk_h q) . c_t      and
//     sum_t p_t (c_t W_uv_h) = (sum_t p_t c_t) W_uv_h,
// so decode is attention in the latent space, shared by every head:
//   1. absorb:     q_lat[b][h] = W_uk_h q[b][h]                (fp32, 512 wide)
//   2. attention:  per (sequence, group of <= 16 heads, partition of the
//                  tokens): online softmax of scale * q_lat . c_t and the
//                  weighted sum of the c_t -> a normalised partial latent
//                  output and its log-sum-exp (the KV-split form, page
//                  "字节跳动 AI Infra (2)", third question, layer-2 table)
//   3. merge + up: o_lat = log-sum-exp merge of the partials (page
//                  "LLM推理优化", section 2.2), out[b][h] = o_lat W_uv_h.
// Step 2 streams the cache (the HBM-bound part); steps 1 and 3 touch only
// the queries, the partials and the two projection matrices.
//
// Attention work-group (4 wavefronts) per piece (sequence b, heads
// 16g .. 16g + 15, partition p); the pieces are dealt persistently (the grid
// holds what the GPU runs at once: two work-groups per CU, each with its own
// 81 KiB of LDS, so one streams while the other waits at a barrier).
// Chunks of 64 tokens are staged in LDS once per work-group (66.5 KiB) and
// used twice:
//   QK  S^T[token][head] = C[token][:] . Q_lat[head][:]   wave w: row groups
//       2 (w % 2) and 2 (w % 2) + 1 (16 tokens each) over latent half w / 2;
//       the two halves' partial scores meet in LDS.  A = 16 latent rows
//       (16-byte LDS reads), B = the wave's half of Q_lat as bf16 hi + lo
//       parts (held in VGPRs).
//   softmax  wave w takes row group w: scales and masks the scores,
//       publishes the row group's maxima, and every wave reads the chunk
//       maximum of each head from LDS (the same value in every wave); then
//       it writes P as bf16 hi + lo parts to LDS and keeps the running sums.
//   PV  O^T[dim][head] += C^T[dim][token] P^T[token][head]   wave w: latent
//       dims 128w .. 128w + 127 over all 64 tokens.  A = C^T, read down the
//       staged rows' columns with gfx950's transposing LDS read
//       (ds_read_b64_tr_b16, two per operand), B = P as bf16 hi + lo from
//       LDS.
// Every wave rescales with the same maxima, so the four dimension slices
// need no merge: each wave writes its own 128 dims of the partial output.
// The latent rows of the next chunk are in flight in VGPRs while one chunk
// is computed (thread t loads rows t / 8 and t / 8 + 32 of it, whole
// 128-byte lines per lane octet).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int DC = kMlaLatentDim;                 // 512
constexpr int NW = 4;                             // wavefronts per attention work-group
constexpr int NT = NW * 64;
constexpr int CT = kMlaChunk;                     // 64 tokens per chunk
constexpr int VPR = DC / 8;                       // 16-byte vectors per latent row: 64
constexpr int VPT = CT * VPR / NT;                // 16-byte vectors per thread per chunk: 8
constexpr int ROW = DC * 2 + 16;                  // LDS bytes per staged row (16 bytes of padding)
constexpr int SPAD = CT + 4;                      // floats per staged score row
constexpr size_t kRowsBytes = static_cast<size_t>(CT) * ROW;
constexpr size_t kScoreBytes = static_cast<size_t>(2) * 16 * SPAD * 4;
static_assert(VPT * NT == CT * VPR, "a chunk is a whole number of vectors per thread");
static_assert(NT / 8 == CT / 2 && VPT == 16, "thread t stages rows t / 8 and t / 8 + 32, vectors t % 8 + 8 i");

// Staged row r keeps its 16-byte vector v at v ^ swz(r): the four 8-row
// groups of a 32-token k-step land on different banks when PV reads down a
// column (rows 8 apart), and the row padding spreads the 16 rows a QK
// row-group reads.
__device__ __forceinline__ int swz(int r) { return ((r >> 3) & 3) << 1; }

constexpr size_t kMlaFixedLds = kRowsBytes + kScoreBytes + static_cast<size_t>(2) * 16 * (CT + 8) * 2 +
                                static_cast<size_t>(4) * 16 * 4 * 2;  // rows, scores, probabilities, maxima/sums

__host__ __device__ constexpr size_t mla_lds_bytes(int tbl_window, int num_seqs) {
  return kMlaFixedLds + static_cast<size_t>(tbl_window) * 4 + static_cast<size_t>(num_seqs + 1) * 4;
}

// gfx950's transposing LDS read of 16-bit elements: within each 16-lane
// group, every lane names 8 bytes (4 elements) and lane t = 4a + b receives
// element b of the lanes a, a + 4, a + 8 and a + 12, in that order (the
// mapping was measured with a probe kernel).  When lane s of a group points
// at 4 consecutive dims d0 + 4 (s % 4) .. of staged row r0 + s / 4, lane t
// receives dim d0 + t of rows r0 .. r0 + 3: four consecutive tokens of one
// dim, half of a matrix-core A operand lane for the PV product.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
__device__ __forceinline__ v4s lds_read_tr16(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p));
}

__device__ __forceinline__ bf16x8 bf16x8_of(const float *x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(x[e]);
  return r;
}

// ---- 1. absorb: q_lat[b][h][c] = sum_d W_uk[c][h * DH + d] q[b][h][d] --------
// On the matrix cores: Q_lat^T[c][b] = W_uk_h[c][:] . Q[b][:] with the 16
// sequences of a work-group as the N dimension (bf16 operands, exact
// products, fp32 sums).  Work-group: head h, 16 sequences, half the latent
// channels (4 wavefronts); wavefront w, counted over both halves, takes
// latent channels 64w .. 64w + 63 (four 16-row tiles).
constexpr int kAbsorbSeqs = 16;
// The latent channels of a (head, 16 sequences) are split over two four-wave
// work-groups, so that the launch covers every CU (the same values; 7.3 ->
// 5.3 us on the benchmark batch, the whole decode 152.1 -> 150.5 us).
constexpr int kAbsorbParts = 2;
constexpr int kAbsorbThreads = DC / kAbsorbParts;

template <int DH>
__global__ __launch_bounds__(kAbsorbThreads) void mla_absorb_kernel(MlaParams p) {
  constexpr int KS = DH / 32;  // k-steps over head_dim
  const uint32_t id = blockIdx.x / kAbsorbParts;
  const int part = static_cast<int>(blockIdx.x % kAbsorbParts);
  const int h = static_cast<int>(id % static_cast<uint32_t>(p.num_heads));
  const int b0 = static_cast<int>(id / static_cast<uint32_t>(p.num_heads)) * kAbsorbSeqs;
  const int lane = threadIdx.x & 63, w = static_cast<int>(threadIdx.x >> 6) + part * (kAbsorbThreads / 64);
  const int m = lane & 15, j = lane >> 4;
  // B operand: lane (sequence m, j) holds q[b0 + m][h][32 s + 8 j ..]
  bf16x8 qb[KS];
  const bool bvalid = b0 + m < p.num_seqs;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (bvalid) v = *reinterpret_cast<const u32x4 *>(p.q + (static_cast<size_t>(b0 + m) * p.num_heads + h) * DH + 32 * s + 8 * j);
    qb[s] = __builtin_bit_cast(bf16x8, v);
  }
  // A operand: lane (channel row m of tile, j) holds W_uk[c][h * DH + 32 s + 8 j ..]
  const size_t wstride = static_cast<size_t>(p.num_heads) * DH;
  u32x4 wa[4][KS];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      wa[t][s] = *reinterpret_cast<const u32x4 *>(p.w_uk + static_cast<size_t>(64 * w + 16 * t + m) * wstride +
                                                   static_cast<size_t>(h) * DH + 32 * s + 8 * j);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[t][s]), qb[s], acc, 0, 0, 0);
    // lane (sequence m, j) holds channels 64 w + 16 t + 4 j + i
    if (bvalid)
      *reinterpret_cast<f32x4 *>(p.q_lat + (static_cast<size_t>(b0 + m) * p.num_heads + h) * DC + 64 * w + 16 * t + 4 * j) = acc;
  }
}

// ---- 2. attention over the latent cache ---------------------------------------

constexpr int PPAD = CT + 8;  // bf16 per staged probability row
constexpr size_t kProbBytes = static_cast<size_t>(2) * 16 * PPAD * 2;  // hi and lo parts
constexpr size_t kStatBytes = static_cast<size_t>(4) * 16 * 4 * 2;      // row-group maxima and sums

struct MlaSmem {
  unsigned char *rows;  // [CT][ROW] staged latent rows (bf16, 16-byte vectors swizzled)
  float *sc;            // [2 halves][16 heads][SPAD] partial scores
  uint16_t *ph, *pl;    // [16 heads][PPAD] probabilities as bf16 hi and lo parts
  float *gmax;          // [4 row groups][16 heads] chunk maxima
  float *gsum;          // [4 row groups][16 heads] final sums
  int32_t *tbl;         // block-table window of the piece
  int32_t *first;       // [num_seqs + 1] first piece of each sequence
};

// Loads of chunk cs: thread t takes latent row t / 8 of the chunk (position
// cs + t / 8, clamped to t1 - 1: rows past the range read a valid row and
// are zeroed when staged) and its 16-byte vectors t % 8 + 8 i: eight loads
// off one address, and every 128-byte line of the row read whole by a lane
// octet.
template <int BS>
__device__ __forceinline__ void mla_issue(u32x4 (&R)[VPT], const MlaParams &p, const int32_t *tbl, int lb0, int cs,
                                          int t1) {
#pragma unroll
  for (int hr = 0; hr < 2; ++hr) {
    const int tok = min(cs + static_cast<int>(threadIdx.x >> 3) + 32 * hr, t1 - 1);
    // out-of-range table entries are clamped so that a bad table can never fault
    const uint32_t pb = min(static_cast<uint32_t>(tbl[tok / BS - lb0]), static_cast<uint32_t>(p.num_blocks - 1));
    const u32x4 *src = reinterpret_cast<const u32x4 *>(p.cache) + (static_cast<size_t>(pb) * BS + tok % BS) * VPR +
                       (threadIdx.x & 7);
#pragma unroll
    for (int i = 0; i < 8; ++i) R[8 * hr + i] = __builtin_nontemporal_load(src + 8 * i);
  }
}

template <int BS>
__device__ __forceinline__ void mla_stage(u32x4 (&R)[VPT], const MlaSmem &sm, int cs, int t1) {
#pragma unroll
  for (int hr = 0; hr < 2; ++hr) {
    const int r = static_cast<int>(threadIdx.x >> 3) + 32 * hr;
    if (cs + CT > t1 && cs + r >= t1) {  // rows past the range: zero, never NaN
#pragma unroll
      for (int i = 0; i < 8; ++i) R[8 * hr + i] = u32x4{0u, 0u, 0u, 0u};
    }
    unsigned char *row = sm.rows + static_cast<size_t>(r) * ROW;
    const int sw = swz(r);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4 *>(row + ((static_cast<int>(threadIdx.x & 7) + 8 * i) ^ sw) * 16) = R[8 * hr + i];
  }
}

struct MlaState {
  f32x4 acc[8];  // O^T[128w + 16n + 4j + i][head m]
  float m_run;   // running maximum (log2 domain), head m (the same in every wave)
  float l_run;   // this lane's share of the running sum of the wave's row group
};

// One chunk staged in LDS: QK (every wave: two row groups over a latent
// half), softmax (wave w: row group w; the chunk maximum through LDS), the
// probabilities through LDS, PV (every wave: its 128 latent dims).
__device__ __forceinline__ void mla_compute(MlaState &st, const MlaSmem &sm, const bf16x8 (&qh)[8],
                                            const bf16x8 (&ql)[8], int cs, int t1, float scale_log2) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int m = lane & 15, j = lane >> 4;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    // QK partial over latent half hf for row group rg
    const int rg = 2 * (w & 1) + rr, hf = w >> 1;
    const int r = 16 * rg + m;
    f32x4 Sh = f32x4{0.f, 0.f, 0.f, 0.f}, Sl = Sh;  // two accumulation chains (hi and lo parts of Q_lat)
    const unsigned char *arow = sm.rows + static_cast<size_t>(r) * ROW;
    const int sw = swz(r);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int v = (32 * hf + 4 * s + j) ^ sw;  // dims 256 hf + 32 s + 8 j ..
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(arow + v * 16));
      Sh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[s], Sh, 0, 0, 0);
      Sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[s], Sl, 0, 0, 0);
    }
    // lane (head m, j) holds tokens 16 rg + 4 j + i
    *reinterpret_cast<f32x4 *>(sm.sc + (hf * 16 + m) * SPAD + 16 * rg + 4 * j) = Sh + Sl;
  }
  lds_barrier();
  f32x4 sv;  // scores (log2 domain) of tokens 16 w + 4 j + i, head m
  {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(sm.sc + m * SPAD + 16 * w + 4 * j);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(sm.sc + (16 + m) * SPAD + 16 * w + 4 * j);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = cs + 16 * w + 4 * j + i < t1 ? (a[i] + b[i]) * scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = max_over_rows(mx);
    if (j == 0) sm.gmax[w * 16 + m] = mx;
  }
  lds_barrier();
  const float cmax = fmaxf(fmaxf(sm.gmax[m], sm.gmax[16 + m]), fmaxf(sm.gmax[32 + m], sm.gmax[48 + m]));
  const float m_new = fmaxf(st.m_run, cmax);        // finite: every chunk holds a position < t1
  const float alpha = fast_exp2(st.m_run - m_new);  // 0 when m_run is -inf
  st.m_run = m_new;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.acc[n] *= alpha;
  {
    float psum = 0.f;
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float p0 = fast_exp2(sv[2 * k] - m_new), p1 = fast_exp2(sv[2 * k + 1] - m_new);
      psum += p0 + p1;
      const __bf16 h0 = static_cast<__bf16>(p0), h1 = static_cast<__bf16>(p1);
      const __bf16 l0 = static_cast<__bf16>(p0 - static_cast<float>(h0));
      const __bf16 l1 = static_cast<__bf16>(p1 - static_cast<float>(h1));
      hi[k] = __builtin_bit_cast(uint16_t, h0) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
      lo[k] = __builtin_bit_cast(uint16_t, l0) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l1)) << 16);
    }
    st.l_run = st.l_run * alpha + psum;
    *reinterpret_cast<u32x2 *>(sm.ph + m * PPAD + 16 * w + 4 * j) = u32x2{hi[0], hi[1]};
    *reinterpret_cast<u32x2 *>(sm.pl + m * PPAD + 16 * w + 4 * j) = u32x2{lo[0], lo[1]};
  }
  lds_barrier();
  // PV over this wave's 128 latent dims
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    // B = P^T: lane (head m, j) takes tokens 32 ks + 8 j .. + 7
    const bf16x8 phi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sm.ph + m * PPAD + 32 * ks + 8 * j));
    const bf16x8 plo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sm.pl + m * PPAD + 32 * ks + 8 * j));
    // A = C^T: lane (dim 128 w + 16 n + m, j) needs rows 32 ks + 8 j + e of its
    // column, e = 0 .. 7.  Two transposing reads: this lane points at row
    // 32 ks + 8 j + m / 4 (then 4 rows further), dims 128 w + 16 n + 4 (m % 4)
    // .. + 3 (8 bytes of a 16-byte vector); all rows of the k-step share the
    // swizzle 2 j.  (Before: eight 32-bit reads down the column and four byte
    // permutes per operand; the whole decode 161.5 -> 159.1 us, bit for bit
    // the same.)
    const unsigned char *trow = sm.rows + static_cast<size_t>(32 * ks + 8 * j + (m >> 2)) * ROW + 8 * (m & 1);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int v = (16 * w + 2 * n + ((m & 3) >> 1)) ^ (2 * j);
      const v4s t0 = lds_read_tr16(trow + v * 16);
      const v4s t1 = lds_read_tr16(trow + 4 * ROW + v * 16);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
      st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, st.acc[n], 0, 0, 0);
      st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, st.acc[n], 0, 0, 0);
    }
  }
}

// One piece: sequence b, heads 16 g .., tokens [part * P, min((part + 1) * P, L)).
template <int BS>
__device__ __forceinline__ void mla_piece(const MlaParams &p, const MlaSmem &sm, int b, int g, int part) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int m = lane & 15, j = lane >> 4;
  const int L = min(max(p.context_lens[b], 0), p.max_blocks_per_seq * BS);
  const int t0 = part * p.partition_size;
  const int t1 = min(t0 + p.partition_size, L);  // > t0: only non-empty pieces are dealt
  const int lb0 = t0 / BS;
  const int nbw = (t1 + BS - 1) / BS - lb0;
  const int32_t *table = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
  __syncthreads();  // the previous piece's readers of the LDS table, rows, scores and sums are done
  for (int i = threadIdx.x; i < nbw; i += NT) sm.tbl[i] = table[lb0 + i];

  // the wave's latent half of its 16 heads' absorbed queries, as bf16 hi + lo
  const int h = 16 * g + m;
  const bool hvalid = h < p.num_heads;
  const int hf = w >> 1;
  bf16x8 qh[8], ql[8];
  {
    const float *qrow = p.q_lat + (static_cast<size_t>(b) * p.num_heads + (hvalid ? h : 0)) * DC + 256 * hf + 8 * j;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float x[8];
      f32x4 u = f32x4{0.f, 0.f, 0.f, 0.f}, v = u;
      if (hvalid) {
        u = *reinterpret_cast<const f32x4 *>(qrow + 32 * s);
        v = *reinterpret_cast<const f32x4 *>(qrow + 32 * s + 4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = u[e];
        x[4 + e] = v[e];
      }
      qh[s] = bf16x8_of(x);
      float r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = x[e] - static_cast<float>(qh[s][e]);
      ql[s] = bf16x8_of(r);
    }
  }
  MlaState st;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  __syncthreads();  // table window staged

  // One chunk in flight ahead of the one computed.  The loads are issued on
  // every path, past the end too (clamped to position t1 - 1: valid rows,
  // never used), so the compiler never has to wait for loads it cannot
  // count.  The barriers inside the loop wait for LDS only, so the loads
  // stay in flight across them.
  const int nch = (t1 - t0 + CT - 1) / CT;
  u32x4 RA[VPT];
  mla_issue<BS>(RA, p, sm.tbl, lb0, t0, t1);
  __builtin_amdgcn_sched_barrier(0);
  for (int k = 0; k < nch; ++k) {
    const int cs = t0 + k * CT;
    lds_barrier();  // the previous chunk's LDS readers are done
    mla_stage<BS>(RA, sm, cs, t1);
    __builtin_amdgcn_sched_barrier(0);
    mla_issue<BS>(RA, p, sm.tbl, lb0, cs + CT, t1);  // past the end: clamped, valid, unused
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // chunk staged
    mla_compute(st, sm, qh, ql, cs, t1, p.scale_log2);
  }

  // the running sum: each wave holds its row group's share (lanes j of a head split them)
  {
    float l = st.l_run + __shfl_xor(st.l_run, 16);
    l = l + __shfl_xor(l, 32);
    if (j == 0) sm.gsum[w * 16 + m] = l;
  }
  __syncthreads();
  const float l = (sm.gsum[m] + sm.gsum[16 + m]) + (sm.gsum[32 + m] + sm.gsum[48 + m]);
  // normalised partial output of this wave's 128 dims, and the log-sum-exp
  if (hvalid) {
    const size_t prow = (static_cast<size_t>(b) * p.num_heads + h) * p.max_num_partitions + part;
    const float inv = 1.f / l;  // l >= 1: the maximum's own term
    float *o = p.part_out + prow * DC + 128 * w + 4 * j;
#pragma unroll
    for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4 *>(o + 16 * n) = st.acc[n] * inv;
    if (w == 0 && j == 0) p.part_lse[prow] = (st.m_run + __log2f(l)) * kLn2;
  }
}

// Persistent pass: work-group g takes pieces g, g + grid, ... of the
// non-empty (sequence, head group, partition) pieces, counted per sequence
// and prefix-summed in LDS.
template <int BS>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void mla_attn_kernel(MlaParams p, int tbl_window) {
  extern __shared__ __align__(16) unsigned char smem[];
  MlaSmem sm;
  sm.rows = smem;
  sm.sc = reinterpret_cast<float *>(smem + kRowsBytes);
  sm.ph = reinterpret_cast<uint16_t *>(smem + kRowsBytes + kScoreBytes);
  sm.pl = sm.ph + 16 * PPAD;
  sm.gmax = reinterpret_cast<float *>(smem + kRowsBytes + kScoreBytes + kProbBytes);
  sm.gsum = sm.gmax + 64;
  sm.tbl = reinterpret_cast<int32_t *>(smem + kRowsBytes + kScoreBytes + kProbBytes + kStatBytes);
  sm.first = sm.tbl + tbl_window;
  static_assert(kRowsBytes + kScoreBytes + kProbBytes + kStatBytes == kMlaFixedLds, "LDS carve");
  const int B = p.num_seqs;
  const int Lmax = p.max_blocks_per_seq * BS;
  const int HG = p.head_groups;
  const int per = (B + NT - 1) / NT;
  const int i0 = min(static_cast<int>(threadIdx.x) * per, B);
  const int i1 = min(i0 + per, B);
  int run = 0;
  for (int i = i0; i < i1; ++i) {
    const int L = min(max(p.context_lens[i], 0), Lmax);
    sm.first[i] = run;
    run += (L + p.partition_size - 1) / p.partition_size * HG;
  }
  __shared__ int32_t wsum[NW];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = incl - run;
  for (int v = 0; v < w; ++v) base += wsum[v];
  int total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) total += wsum[v];
  for (int i = i0; i < i1; ++i) sm.first[i] += base;
  if (threadIdx.x == 0) sm.first[B] = total;
  __syncthreads();

  for (int piece = blockIdx.x; piece < total; piece += gridDim.x) {
    int lo = 0, hi = B;  // first[lo] <= piece < first[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sm.first[mid] <= piece)
        lo = mid;
      else
        hi = mid;
    }
    const int local = piece - sm.first[lo];
    const int nparts = (sm.first[lo + 1] - sm.first[lo]) / HG;
    if (nparts > 0) mla_piece<BS>(p, sm, lo, local / nparts, local % nparts);
  }
}

// ---- 3. merge the partitions and up-project, on the matrix cores -----------------
// Work-group: head h, kUmSeqs sequences, 256 threads.
//   merge: thread (sequence bb = t / 32, channels 16 (t % 32) ..): o_lat =
//          sum_p e^{lse_p - M} o_p / sum_p e^{lse_p - M} (partitions in
//          order), kept in LDS as bf16 hi + lo rows (the A operand: rows of
//          sequences; rows kUmSeqs .. 15 zero).
//   up:    out[b][h][:] = o_lat W_uv,h on 16x16x32 MFMAs: wave w takes the
//          output dims 16 (NTW w + nt) ..; W_uv's rows staged in LDS 64 at a
//          time (the next chunk's loads in flight), its columns read with the
//          transposing LDS read (the B operand: 8 channels of one dim per lane).
// (Before: the up-projection on the vector ALUs, W_uv read from LDS one
// element per product: 19.9 us on the benchmark batch, its waves held at the
// staging barriers; now the whole decode 158.6 -> 152.2 us.)
constexpr int kUmSeqs = 8;
constexpr int kUmThreads = 256;
constexpr int kUmRows = 64;
constexpr int kOPad = DC + 8;  // bf16 per staged o_lat row

template <int DH>
__global__ __launch_bounds__(kUmThreads) void mla_merge_up_kernel(MlaParams p) {
  constexpr int WROW = DH + 16;                       // bf16 per staged W_uv row (32 bytes of padding)
  constexpr int VPW = DH / 8;                         // 16-byte vectors per W_uv row slice
  constexpr int WV = kUmRows * VPW / kUmThreads;      // vectors per thread per chunk
  constexpr int NTW = DH / 64;                        // 16-dim output tiles per wave
  static_assert(WV * kUmThreads == kUmRows * VPW && NTW >= 1, "shapes");
  __shared__ __align__(16) uint16_t oh[16][kOPad];
  __shared__ __align__(16) uint16_t ol[16][kOPad];
  __shared__ __align__(16) uint16_t wl[2][kUmRows][WROW];
  const int h = static_cast<int>(blockIdx.x % static_cast<uint32_t>(p.num_heads));
  const int b0 = static_cast<int>(blockIdx.x / static_cast<uint32_t>(p.num_heads)) * kUmSeqs;
  const int nb = min(kUmSeqs, p.num_seqs - b0);
  const int Lmax = p.max_blocks_per_seq * p.block_size;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, m = lane & 15, j = lane >> 4;
  const size_t wstride = static_cast<size_t>(p.num_heads) * DH;
  const uint16_t *wbase = p.w_uv + static_cast<size_t>(h) * DH;

  u32x4 wr[WV];
  auto issue_w = [&](int c0) {
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int v = t + kUmThreads * i;
      wr[i] = *reinterpret_cast<const u32x4 *>(wbase + static_cast<size_t>(c0 + v / VPW) * wstride + (v % VPW) * 8);
    }
  };
  auto stage_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int v = t + kUmThreads * i;
      *reinterpret_cast<u32x4 *>(&wl[buf][v / VPW][(v % VPW) * 8]) = wr[i];
    }
  };
  issue_w(0);

  {
    const int bb = t / 32, c0 = (t % 32) * 16;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    float l = 0.f;
    if (bb < nb) {
      const int b = b0 + bb;
      const int L = min(max(p.context_lens[b], 0), Lmax);
      const int n = min((L + p.partition_size - 1) / p.partition_size, p.max_num_partitions);
      const size_t row = (static_cast<size_t>(b) * p.num_heads + h) * p.max_num_partitions;
      float M = -INFINITY;
      for (int q = 0; q < n; ++q) M = fmaxf(M, p.part_lse[row + q]);
#pragma unroll 2
      for (int q = 0; q < n; ++q) {
        const float wt = fast_exp2((p.part_lse[row + q] - M) * 1.4426950408889634f);
        l += wt;
        const f32x4 *src = reinterpret_cast<const f32x4 *>(p.part_out + (row + q) * DC + c0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const f32x4 x = src[v];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[4 * v + i] += wt * x[i];
        }
      }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;  // L = 0: a zero row
    u32x4 hv[2], lv[2];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float o0 = acc[e] * inv, o1 = acc[e + 1] * inv;
      const __bf16 h0 = static_cast<__bf16>(o0), h1 = static_cast<__bf16>(o1);
      const __bf16 l0 = static_cast<__bf16>(o0 - static_cast<float>(h0));
      const __bf16 l1 = static_cast<__bf16>(o1 - static_cast<float>(h1));
      hv[e >> 3][(e >> 1) & 3] = __builtin_bit_cast(uint16_t, h0) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
      lv[e >> 3][(e >> 1) & 3] = __builtin_bit_cast(uint16_t, l0) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l1)) << 16);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      *reinterpret_cast<u32x4 *>(&oh[bb][c0 + 8 * k]) = hv[k];
      *reinterpret_cast<u32x4 *>(&ol[bb][c0 + 8 * k]) = lv[k];
      // the padding rows of the A operand
      *reinterpret_cast<u32x4 *>(&oh[kUmSeqs + bb][c0 + 8 * k]) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(&ol[kUmSeqs + bb][c0 + 8 * k]) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  static_assert(kUmSeqs == 8, "the padding rows are written by the merge threads");
  stage_w(0);

  f32x4 acc[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int NCH = DC / kUmRows;
  for (int k = 0; k < NCH; ++k) {
    const int buf = k & 1;
    if (k + 1 < NCH) issue_w((k + 1) * kUmRows);
    lds_barrier();  // chunk k staged (and, the first time, the o_lat rows)
#pragma unroll
    for (int ks = 0; ks < kUmRows / 32; ++ks) {
      const int cb = k * kUmRows + 32 * ks;
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&oh[m][cb + 8 * j]));
      const bf16x8 alo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&ol[m][cb + 8 * j]));
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int d0 = 16 * (NTW * w + nt);
        const unsigned char *src =
            reinterpret_cast<const unsigned char *>(&wl[buf][32 * ks + 8 * j + (m >> 2)][d0 + 4 * (m & 3)]);
        const v4s t0 = lds_read_tr16(src);
        const v4s t1 = lds_read_tr16(src + 4 * WROW * 2);
        const bf16x8 bw = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bw, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bw, acc[nt], 0, 0, 0);
      }
    }
    if (k + 1 < NCH) stage_w(buf ^ 1);  // its readers (chunk k - 1) passed this chunk's barrier
  }
  // lane (dim m of the tile, j) holds sequences 4 j .. 4 j + 3
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int d = 16 * (NTW * w + nt) + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bb = 4 * j + i;
      if (bb < nb) {
        const size_t idx = (static_cast<size_t>(b0 + bb) * p.num_heads + h) * DH + d;
        if (p.out_bf16)
          static_cast<uint16_t *>(p.out)[idx] = float_to_bf16_bits(acc[nt][i]);
        else
          static_cast<float *>(p.out)[idx] = acc[nt][i];
      }
    }
  }
}

// ---- latent append: one wavefront per token row (1 KiB) ------------------------
__global__ __launch_bounds__(256) void mla_append_kernel(MlaAppendParams p) {
  const int t = static_cast<int>(blockIdx.x) * 4 + static_cast<int>(threadIdx.x >> 6);
  if (t >= p.num_tokens) return;
  const int32_t s = p.slot_mapping[t];
  if (s < 0 || static_cast<int64_t>(s) >= static_cast<int64_t>(p.num_blocks) * p.block_size) return;
  const int lane = threadIdx.x & 63;
  const u32x4 v = reinterpret_cast<const u32x4 *>(p.rows)[static_cast<size_t>(t) * VPR + lane];
  reinterpret_cast<u32x4 *>(p.cache)[static_cast<size_t>(s) * VPR + lane] = v;
}

template <int BS>
hipError_t launch_attn(const MlaParams &p, hipStream_t s) {
  const int tw = p.partition_size / BS;
  const size_t lds = mla_lds_bytes(tw, p.num_seqs);
  auto kern = mla_attn_kernel<BS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  int per_cu = 0, dev = 0, cus = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), NT, lds);
  if (e != hipSuccess) return e;
  const int64_t most = static_cast<int64_t>(p.num_seqs) * p.head_groups * p.max_num_partitions;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(static_cast<int64_t>(std::max(per_cu, 1)) * cus, most));
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(grid)), dim3(NT), lds, s, p, tw);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_dh(const MlaParams &p, hipStream_t s) {
  const uint32_t groups = static_cast<uint32_t>((p.num_seqs + kAbsorbSeqs - 1) / kAbsorbSeqs);
  hipLaunchKernelGGL(mla_absorb_kernel<DH>, dim3(groups * static_cast<uint32_t>(p.num_heads) * kAbsorbParts),
                     dim3(kAbsorbThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (p.block_size) {
    case 16: e = launch_attn<16>(p, s); break;
    case 32: e = launch_attn<32>(p, s); break;
    case 64: e = launch_attn<64>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const uint32_t ugroups = static_cast<uint32_t>((p.num_seqs + kUmSeqs - 1) / kUmSeqs);
  hipLaunchKernelGGL(mla_merge_up_kernel<DH>, dim3(ugroups * static_cast<uint32_t>(p.num_heads)),
                     dim3(kUmThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_decode(const MlaParams &p, hipStream_t s) {
  if (p.head_dim == 128) return launch_dh<128>(p, s);
  if (p.head_dim == 64) return launch_dh<64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_mla_append(const MlaAppendParams &p, hipStream_t s) {
  const uint32_t nwg = static_cast<uint32_t>((p.num_tokens + 3) / 4);
  hipLaunchKernelGGL(mla_append_kernel, dim3(nwg), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
