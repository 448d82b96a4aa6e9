// Paged attention in fp32 (small fp32 streams).
//
// Same operation as the bf16 kernels: O = softmax(s * Q K^T) V over the
// tokens of a sequence's page-table entries, no mask ("LingBot-Map Paged KV
// Cache", section 2), with an online softmax over 64-key tiles.  fp32 inputs,
// fp32 products and fp32 accumulation, on the matrix cores
// (v_mfma_f32_32x32x2_f32: a 32x32 block, two steps of the contracted index
// per instruction).
//
// A workgroup is two waves; each wave owns 32 query rows, so a workgroup
// covers 64 rows of one (sequence, head, key split).  (Four-wave, 128-row
// workgroups measured 12% slower on a 262-query stream: coarser tiles leave
// more rows idle and fewer workgroups to balance over the CUs.)  Per 64-key tile a wave
// forms S^T = K Q^T (two 32-key blocks, 32 steps over the 64 dims each), the
// softmax against a running maximum taken per tile, and O^T += V^T P^T (two
// 32-dim blocks, 32 steps over the 64 keys each).
//
// Operand layout of a 32x32x2 product: lane l supplies row (or column) l % 32
// at step index l / 32.  The score products give each lane the dims
// 32 * (l / 32) .. +31 of its query (Q in registers) and of its key (K read
// from LDS as float4).  A 32x32 accumulator leaves lane l holding column
// l % 32 at rows (r / 4) * 8 + 4 * (l / 32) + r % 4, r = 0..15; the P V
// products take exactly those keys as their step index, so the probabilities
// feed the next products from the registers they were formed in, and V^T is
// read as float4 runs of 4 consecutive keys.
//
// Tiles go through LDS in two buffers: K as [key][dim] and V^T as [dim][key],
// each row's 16-byte chunks XOR-swizzled by the row index so that the 32 rows
// a product reads fall on distinct banks.  The next tile's global loads are
// issued into registers before the current tile's products, so they overlap.
// V values of keys past a page's valid length are stored as zeros and their
// scores set to -inf, whatever the pool holds there.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace kvc {
namespace {

typedef float floatx16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int D = kHeadDim;
constexpr int KT = kKeyTile;
constexpr int W = 2;          // waves per workgroup
constexpr int ROWS = W * 32;  // query rows per workgroup
constexpr int NT = W * 64;    // threads
constexpr int TILE = KT * D;  // floats of K (or of V^T) per tile
constexpr int CPT = TILE / 4 / NT;  // float4 chunks of K (and of V) each thread stages per tile

// Maximum and sum of x over lanes l and l ^ 32 (the two halves of a query's
// keys).  The swap returns the lane's own value and its partner's, one in
// each element; max and sum do not depend on which is which.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Position of 16-byte chunk c of LDS row r (16 chunks per row).
__device__ __forceinline__ int swz_chunk(int r, int c) { return c ^ (r & 15); }

// The tile sequence of one key split: table entries [e, ee), 64-key tiles of
// each entry's valid length (entries of length 0 are skipped).
struct TileCursor {
  int e, pid, len, kt;
};

template <class Src>
__device__ __forceinline__ void cursor_skip_empty(const Src& src, int ee, TileCursor& c) {
  while (c.e < ee) {
    attn_entry(src, c.e, c.pid, c.len);
    if (c.len > 0) return;
    ++c.e;
  }
}

template <class Src>
__device__ __forceinline__ void cursor_advance(const Src& src, int ee, TileCursor& c) {
  ++c.kt;
  if (c.kt * KT >= c.len) {
    c.kt = 0;
    ++c.e;
    cursor_skip_empty(src, ee, c);
  }
}

template <class Src>
__global__ __launch_bounds__(NT) void attn_f32_kernel(const Src src) {
  const AttnParams& p = attn_base(src);
  __shared__ __attribute__((aligned(16))) float lds[2][2][TILE];  // [buffer][K, V^T][row * 64 + dim or key]

  // ---- which (sequence, head, split, query tile) --------------------------
  int g, qt;
  attn_tile_of(p, blockIdx.x, g, qt);
  if (g >= p.groups) return;
  const int split = g % p.num_splits;
  const int sh = g / p.num_splits;
  const int h = sh % p.num_heads;
  const int seq = sh / p.num_heads;
  int q0, qn, ebase, ecount;
  attn_seq(src, seq, q0, qn, ebase, ecount);
  const int row0 = qt * ROWS;
  if (row0 >= qn) return;
  const int per = (ecount + p.num_splits - 1) / p.num_splits;
  const int eb = ebase + min(ecount, split * per);
  const int ee = ebase + min(ecount, (split + 1) * per);

  const int H = p.num_heads;
  const int P = p.page_size;
  const float sl2 = p.scale_log2;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;  // query column of the accumulators; K / V^T row of the operands
  const int lh = lane >> 5;  // step index within a product
  const int wrow0 = row0 + wave * 32;
  const bool active = wrow0 < qn;  // wave-uniform; idle waves still stage tiles and synchronise

  const float* __restrict__ qg = static_cast<const float*>(p.q);
  const float* __restrict__ kg = static_cast<const float*>(p.k_pool);
  const float* __restrict__ vg = static_cast<const float*>(p.v_pool);

  // ---- queries -> registers: q[t] = Q[row][32 * lh + t] (rows past the
  // sequence repeat its last row; their outputs are never written).
  float q[32];
  {
    const int row = min(wrow0 + lr, qn - 1);
    const float4* qp = reinterpret_cast<const float4*>(qg + (static_cast<size_t>(q0 + row) * H + h) * D + lh * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = qp[i];
      q[4 * i] = v.x;
      q[4 * i + 1] = v.y;
      q[4 * i + 2] = v.z;
      q[4 * i + 3] = v.w;
    }
  }

  // ---- staging: thread tid moves chunks tid + NT * i (row = chunk / 16,
  // 16-byte chunk = chunk % 16) of the tile's K rows and of its V^T rows.
  // (held as 16-float vectors: as arrays of float4 they were moved to LDS)
  static_assert(CPT % 4 == 0, "staging vectors hold four chunks each");
  floatx16 rk[CPT / 4], rv[CPT / 4];
  auto load_tile = [&](const TileCursor& c) {
    const float* kb = kg + ((static_cast<size_t>(c.pid) * H + h) * P + static_cast<size_t>(c.kt) * KT) * D;
    const float* vb = vg + (static_cast<size_t>(c.pid) * H + h) * D * P + static_cast<size_t>(c.kt) * KT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + NT * i;
      const int row = ci >> 4, ch = ci & 15;
      const float4 kv = *reinterpret_cast<const float4*>(kb + row * D + ch * 4);
      const float4 vv = *reinterpret_cast<const float4*>(vb + static_cast<size_t>(row) * P + ch * 4);
      rk[i >> 2][4 * (i & 3)] = kv.x;
      rk[i >> 2][4 * (i & 3) + 1] = kv.y;
      rk[i >> 2][4 * (i & 3) + 2] = kv.z;
      rk[i >> 2][4 * (i & 3) + 3] = kv.w;
      rv[i >> 2][4 * (i & 3)] = vv.x;
      rv[i >> 2][4 * (i & 3) + 1] = vv.y;
      rv[i >> 2][4 * (i & 3) + 2] = vv.z;
      rv[i >> 2][4 * (i & 3) + 3] = vv.w;
    }
  };
  auto store_tile = [&](float* lk, float* lv, int nk) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + NT * i;
      const int row = ci >> 4, ch = ci & 15;
      *reinterpret_cast<float4*>(lk + row * D + swz_chunk(row, ch) * 4) =
          make_float4(rk[i >> 2][4 * (i & 3)], rk[i >> 2][4 * (i & 3) + 1], rk[i >> 2][4 * (i & 3) + 2], rk[i >> 2][4 * (i & 3) + 3]);
      // Pool chunk ch of a V^T row holds slots v_slot_pos(4 ch) .. +3, i.e.
      // the keys of chunk kc = ch with its two low bits swapped, in order.
      const int kc = (ch & ~3) | ((ch & 1) << 1) | ((ch >> 1) & 1);
      float4 v = make_float4(rv[i >> 2][4 * (i & 3)], rv[i >> 2][4 * (i & 3) + 1], rv[i >> 2][4 * (i & 3) + 2], rv[i >> 2][4 * (i & 3) + 3]);
      const int k0 = kc * 4;
      if (k0 + 0 >= nk) v.x = 0.f;
      if (k0 + 1 >= nk) v.y = 0.f;
      if (k0 + 2 >= nk) v.z = 0.f;
      if (k0 + 3 >= nk) v.w = 0.f;
      *reinterpret_cast<float4*>(lv + row * KT + swz_chunk(row, kc) * 4) = v;
    }
  };

  float m_run = -INFINITY;  // running maximum of scaled scores (log2 domain), per query
  float l_run = 0.f;        // this lane's partial row sum
  floatx16 o0 = {}, o1 = {};  // O^T, dims 0..31 and 32..63

  auto compute = [&](const float* lk, const float* lv, int nk) {
    // S^T = K Q^T: s0 keys 0..31, s1 keys 32..63; step t = 4 gi + i is dim 32 lh + t.
    floatx16 s0 = {}, s1 = {};
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
      const int c = lh * 8 + gi;
      const float4 ka = *reinterpret_cast<const float4*>(lk + lr * D + swz_chunk(lr, c) * 4);
      const float4 kb = *reinterpret_cast<const float4*>(lk + (32 + lr) * D + swz_chunk(lr, c) * 4);
      s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka.x, q[4 * gi + 0], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kb.x, q[4 * gi + 0], s1, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka.y, q[4 * gi + 1], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kb.y, q[4 * gi + 1], s1, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka.z, q[4 * gi + 2], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kb.z, q[4 * gi + 2], s1, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(ka.w, q[4 * gi + 3], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kb.w, q[4 * gi + 3], s1, 0, 0, 0);
    }
    // element r of s0 is key (r / 4) * 8 + 4 lh + r % 4; s1 adds 32
    if (nk < KT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + 4 * lh + (r & 3);
        if (key >= nk) s0[r] = -INFINITY;
        if (key + 32 >= nk) s1[r] = -INFINITY;
      }
    }
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mx[i] = fmaxf(fmaxf(fmaxf(s0[i], s0[i + 4]), fmaxf(s0[i + 8], s0[i + 12])),
                    fmaxf(fmaxf(s1[i], s1[i + 4]), fmaxf(s1[i + 8], s1[i + 12])));
    float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    mt = pair_max(mt);
    // every tile holds at least one valid key, so m_new is finite for finite data
    const float m_new = fmaxf(m_run, mt * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    const float nm = -m_new;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, nm));
      s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, nm));
      ps[r & 3] += s0[r] + s1[r];
    }
    l_run = __builtin_fmaf(l_run, alpha, (ps[0] + ps[1]) + (ps[2] + ps[3]));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= alpha;
      o1[r] *= alpha;
    }
    // O^T += V^T P^T: key group a (keys 8a + 4 lh + b, b = 0..3) is V^T chunk
    // 2a + lh and P elements 4a + b of s0 (a < 4) or 4(a - 4) + b of s1.
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int c = 2 * a + lh;
      const float4 va = *reinterpret_cast<const float4*>(lv + lr * KT + swz_chunk(lr, c) * 4);
      const float4 vb = *reinterpret_cast<const float4*>(lv + (32 + lr) * KT + swz_chunk(lr, c) * 4);
      const float p0 = a < 4 ? s0[4 * a + 0] : s1[4 * (a - 4) + 0];
      const float p1 = a < 4 ? s0[4 * a + 1] : s1[4 * (a - 4) + 1];
      const float p2 = a < 4 ? s0[4 * a + 2] : s1[4 * (a - 4) + 2];
      const float p3 = a < 4 ? s0[4 * a + 3] : s1[4 * (a - 4) + 3];
      o0 = __builtin_amdgcn_mfma_f32_32x32x2f32(va.x, p0, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x2f32(vb.x, p0, o1, 0, 0, 0);
      o0 = __builtin_amdgcn_mfma_f32_32x32x2f32(va.y, p1, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x2f32(vb.y, p1, o1, 0, 0, 0);
      o0 = __builtin_amdgcn_mfma_f32_32x32x2f32(va.z, p2, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x2f32(vb.z, p2, o1, 0, 0, 0);
      o0 = __builtin_amdgcn_mfma_f32_32x32x2f32(va.w, p3, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x2f32(vb.w, p3, o1, 0, 0, 0);
    }
  };

  // ---- key loop: tile j in buffer j % 2.  The buffer written at iteration j
  // was last read at iteration j - 2, which every wave finished before the
  // barrier of iteration j - 1.
  TileCursor cur{eb, 0, 0, 0};
  cursor_skip_empty(src, ee, cur);
  if (cur.e < ee) load_tile(cur);
  int buf = 0;
  while (cur.e < ee) {
    const int nk = min(KT, cur.len - cur.kt * KT);
    float* lk = lds[buf][0];
    float* lv = lds[buf][1];
    store_tile(lk, lv, nk);
    __syncthreads();
    TileCursor nx = cur;
    cursor_advance(src, ee, nx);
    if (nx.e < ee) load_tile(nx);
    if (active) compute(lk, lv, nk);
    cur = nx;
    buf ^= 1;
  }

  // ---- epilogue --------------------------------------------------------------
  if (!active) return;
  const int qrow = wrow0 + lr;
  const float ltot = pair_sum(l_run);
  if (qrow >= qn) return;
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse_nat = empty ? -INFINITY : (m_run + __log2f(ltot)) * 0.69314718055994530942f;
  const size_t orow = static_cast<size_t>(q0 + qrow) * H + h;
  float* out = p.num_splits == 1 ? static_cast<float*>(p.o) + orow * D
                                 : p.part_o + (static_cast<size_t>(split) * p.total_q * H + orow) * D;
  // element r of o0 is dim (r / 4) * 8 + 4 lh + r % 4; o1 adds 32
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    *reinterpret_cast<float4*>(out + 8 * a + 4 * lh) =
        make_float4(o0[4 * a] * inv, o0[4 * a + 1] * inv, o0[4 * a + 2] * inv, o0[4 * a + 3] * inv);
    *reinterpret_cast<float4*>(out + 32 + 8 * a + 4 * lh) =
        make_float4(o1[4 * a] * inv, o1[4 * a + 1] * inv, o1[4 * a + 2] * inv, o1[4 * a + 3] * inv);
  }
  if (lh == 0) {
    if (p.num_splits == 1) {
      if (p.lse) p.lse[orow] = lse_nat;
    } else {
      p.part_lse[static_cast<size_t>(split) * p.total_q * H + orow] = lse_nat;
    }
  }
}

}  // namespace

int attn_f32_rows_per_tile() { return ROWS; }

template <class Src>
static hipError_t launch_impl(const Src& src, hipStream_t stream) {
  const AttnParams& p = attn_base(src);
  const dim3 grid(static_cast<unsigned>(p.q_tiles) * p.groups_padded);
  hipLaunchKernelGGL((attn_f32_kernel<Src>), grid, dim3(NT), 0, stream, src);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) { return launch_impl(p, stream); }
hipError_t launch_attn_f32(const AttnParamsInline& p, hipStream_t stream) { return launch_impl(p, stream); }

}  // namespace kvc
