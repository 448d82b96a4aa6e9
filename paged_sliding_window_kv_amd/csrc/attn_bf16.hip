// Paged attention, bf16 inputs, fp32 accumulation, for CDNA4 (gfx950).
//
// Computes O = softmax(s * Q K^T) V for each query sequence and head over the
// tokens of the sequence's page-table entries, with no mask: the visible
// table already lists exactly the tokens a frame or chunk attends to, and
// each page carries its valid length ("LingBot-Map Paged KV Cache", section
// 2; "vLLM-Omni RFC #2727", section 1: global attention over the window).
// The online softmax processes one 64-key tile at a time and keeps a running
// maximum and sum per query, so no score matrix is stored.
//
// Mapping to the hardware
//  * One workgroup = NW waves = NW*32 query rows of one (sequence, head,
//    key split).  Each wave owns 32 query rows; its Q fragment stays in
//    registers for the whole key loop.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims from LDS, B = 16 dims x
//    32 queries from registers.  In the 32x32 accumulator each lane then
//    holds 16 scores of a single query, so the row maximum and row sum are
//    in-lane reductions plus one exchange between lane l and lane l + 32.
//  * The probabilities are reused in registers as the B operand of
//    O^T = V^T P^T (A = 32 dims x 16 keys of V^T from LDS).  Which k-slot of
//    the instruction carries which key is free (k is summed over), so the
//    key order of the accumulator layout is used as is and V^T is written to
//    LDS in the matching order: each 16-byte LDS chunk of a V^T row holds
//    keys {4h..4h+3, 8+4h..8+4h+3} of a 16-key group for half-wave h.
//  * V is stored transposed in the pool ([dim][slot] per page and head), so
//    a V^T tile row is 128 contiguous bytes of HBM.
//  * K and V^T tiles (8 KiB each) are double-buffered in LDS; the next
//    tile's global loads are issued before the current tile's products.
//    16-byte chunks are XOR-swizzled by row so that the fragment reads of 8
//    consecutive rows fall in distinct banks.
//  * Keys past a page's valid length: scores are set to -inf and V^T is
//    written as zeros, so stale pool contents (even NaN) never reach O.
//  * The 1-D grid is ordered so that all query tiles of one (sequence, head,
//    split) share the same index modulo 8 and therefore the same XCD (and its
//    L2), which serves their repeated reads of that head's K/V.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float floatx16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float floatx8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int D = kHeadDim;        // 64
constexpr int KT = kKeyTile;       // 64 keys per tile
constexpr int TILE_ELEMS = KT * D; // 4096 bf16 = 8 KiB
constexpr int TILE_CHUNKS = TILE_ELEMS / 8;  // 512 chunks of 16 bytes

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base, int row, int chunk) {
  // 128-byte rows, 16-byte chunks swizzled by row.
  return *reinterpret_cast<const bf16x8*>(base + row * D + ((chunk ^ (row & 7)) << 3));
}

__device__ __forceinline__ bf16x8 to_bf16x8(floatx16 s, int base) {
  floatx8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = s[base + j];
  return __builtin_convertvector(f, bf16x8);
}

__device__ __forceinline__ uint4 zero_keys(uint4 v, int first_key, int nk) {
  // Zero the bf16 lanes whose key index (first_key + i) is >= nk.
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k0 = first_key + 2 * i;
    if (k0 >= nk) w[i] = 0u;
    else if (k0 + 1 >= nk) w[i] &= 0xFFFFu;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(const AttnParams p) {
  constexpr int NT = NW * 64;
  constexpr int ROWS = NW * 32;
  constexpr int CPT = (TILE_CHUNKS + NT - 1) / NT;  // 16-byte chunks per thread per tensor
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][TILE_ELEMS];

  // ---- which (sequence, head, split, query tile) ----------------------------
  const int L = blockIdx.x;
  const int g = L % p.groups_padded;
  const int qt = L / p.groups_padded;
  if (g >= p.groups) return;
  const int split = g % p.num_splits;
  const int sh = g / p.num_splits;
  const int h = sh % p.num_heads;
  const int seq = sh / p.num_heads;
  const int q0 = p.qo_indptr[seq];
  const int qn = p.qo_indptr[seq + 1] - q0;
  const int row0 = qt * ROWS;
  if (row0 >= qn) return;
  const int ebase = p.kv_indptr[seq];
  const int ecount = p.kv_indptr[seq + 1] - ebase;
  const int per = (ecount + p.num_splits - 1) / p.num_splits;
  const int eb = ebase + min(ecount, split * per);
  const int ee = ebase + min(ecount, (split + 1) * per);

  const int H = p.num_heads;
  const int P = p.page_size;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int wrow0 = row0 + wave * 32;
  const bool active = wrow0 < qn;
  const int qrow = wrow0 + lr;
  const bool qvalid = qrow < qn;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k_pool);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v_pool);

  // ---- Q fragment (B operand of S^T = K Q^T): Q[row][16*st + 8*lh .. +7] ----
  bf16x8 qf[4];
  {
    const uint16_t* qp = qg + (static_cast<size_t>(q0 + (qvalid ? qrow : 0)) * H + h) * D + 8 * lh;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * st) : make_uint4(0, 0, 0, 0);
      qf[st] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- tile cursor over the split's table entries --------------------------
  auto entry = [&](int e, int& pid, int& len) {
    pid = p.page_ids[e];
    len = p.page_lens[e];
    len = len < 0 ? 0 : (len > P ? P : len);
    if (pid < 0 || pid >= p.num_pool_pages) len = 0;
  };
  int ce = eb, ckt = 0, clen = 0, cpid = 0;
  while (ce < ee) {
    entry(ce, cpid, clen);
    if (clen > 0) break;
    ++ce;
  }
  bool have = ce < ee;

  uint4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int pid, int kt) {
    const uint16_t* kb = kg + ((static_cast<size_t>(pid) * H + h) * P + kt * KT) * D;
    const uint16_t* vb = vg + (static_cast<size_t>(pid) * H + h) * D * P + kt * KT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CPT * NT == TILE_CHUNKS || c < TILE_CHUNKS) {
        kreg[i] = *reinterpret_cast<const uint4*>(kb + c * 8);                       // key c/8, dims (c%8)*8
        vreg[i] = *reinterpret_cast<const uint4*>(vb + (c >> 3) * P + (c & 7) * 8);  // dim c/8, keys (c%8)*8
      }
    }
  };
  auto store_tile = [&](int buf, int nk) {
    uint16_t* lk = lds_k[buf];
    uint16_t* lv = lds_v[buf];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CPT * NT == TILE_CHUNKS || c < TILE_CHUNKS) {
        const int row = c >> 3, ch = c & 7;
        *reinterpret_cast<uint4*>(lk + row * D + ((ch ^ (row & 7)) << 3)) = kreg[i];
        uint4 v = vreg[i];
        if (nk < KT) v = zero_keys(v, ch * 8, nk);
        // logical keys 8ch..8ch+7 = 16g + 8e + {0..7}: low half -> physical chunk 2g,
        // high half -> physical chunk 2g+1, both at half e.
        const int gg = ch >> 1, e = ch & 1;
        uint2* r = reinterpret_cast<uint2*>(lv + row * D);
        r[((2 * gg) ^ (row & 7)) * 2 + e] = make_uint2(v.x, v.y);
        r[((2 * gg + 1) ^ (row & 7)) * 2 + e] = make_uint2(v.z, v.w);
      }
    }
  };

  float m_run = -INFINITY;  // running max of scaled scores (log2 domain)
  float l_run = 0.f;        // this lane's partial row sum
  floatx16 o0 = {}, o1 = {};

  if (have) {
    load_tile(cpid, 0);
    store_tile(0, min(KT, clen));
    __syncthreads();
  }
  int buf = 0;
  while (have) {
    const int nk = min(KT, clen - ckt * KT);
    // advance the cursor
    int ne = ce, nkt = ckt + 1, nlen = clen, npid = cpid;
    if (nkt * KT >= nlen) {
      nkt = 0;
      ++ne;
      while (ne < ee) {
        entry(ne, npid, nlen);
        if (nlen > 0) break;
        ++ne;
      }
    }
    const bool next = ne < ee;
    if (next) load_tile(npid, nkt);

    if (active) {
      const uint16_t* lk = lds_k[buf];
      const uint16_t* lv = lds_v[buf];
      floatx16 s0 = {}, s1 = {};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 a0 = lds_frag(lk, lr, 2 * st + lh);
        const bf16x8 a1 = lds_frag(lk, 32 + lr, 2 * st + lh);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[st], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[st], s1, 0, 0, 0);
      }
      if (nk < KT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
          if (key >= nk) s0[r] = -INFINITY;
          if (key + 32 >= nk) s1[r] = -INFINITY;
        }
      }
      float mx = s0[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * p.scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], p.scale_log2, -m_new));
        s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], p.scale_log2, -m_new));
        rs += s0[r] + s1[r];
      }
      l_run = __builtin_fmaf(l_run, alpha, rs);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o0[r] *= alpha;
        o1[r] *= alpha;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 pb = to_bf16x8(t < 2 ? s0 : s1, 8 * (t & 1));
        const bf16x8 va0 = lds_frag(lv, lr, 2 * t + lh);
        const bf16x8 va1 = lds_frag(lv, 32 + lr, 2 * t + lh);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va0, pb, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va1, pb, o1, 0, 0, 0);
      }
    }
    if (!next) break;
    store_tile(buf ^ 1, min(KT, nlen - nkt * KT));
    __syncthreads();
    buf ^= 1;
    ce = ne;
    ckt = nkt;
    clen = nlen;
    cpid = npid;
  }

  if (!active) return;
  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float lse_nat = empty ? -INFINITY : (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  if (!qvalid) return;
  const size_t orow = static_cast<size_t>(q0 + qrow) * H + h;
  if (p.num_splits == 1) {
    uint16_t* og = static_cast<uint16_t*>(p.o) + orow * D;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        floatx4 f;
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = (db ? o1 : o0)[r4 * 4 + j] * inv;
        const bf16x4 b = __builtin_convertvector(f, bf16x4);
        *reinterpret_cast<bf16x4*>(og + db * 32 + r4 * 8 + lh * 4) = b;
      }
    }
    if (p.lse && lh == 0) p.lse[orow] = lse_nat;
  } else {
    float* po = p.part_o + (static_cast<size_t>(split) * p.total_q * H + orow) * D;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        floatx4 f;
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = (db ? o1 : o0)[r4 * 4 + j] * inv;
        *reinterpret_cast<floatx4*>(po + db * 32 + r4 * 8 + lh * 4) = f;
      }
    }
    if (lh == 0) p.part_lse[static_cast<size_t>(split) * p.total_q * H + orow] = lse_nat;
  }
}

}  // namespace

int attn_bf16_rows_per_tile(int waves) { return waves * 32; }

hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(p.q_tiles) * p.groups_padded);
  switch (waves) {
    case 4:
      hipLaunchKernelGGL(attn_bf16_kernel<4>, grid, dim3(256), 0, stream, p);
      break;
    case 8:
      hipLaunchKernelGGL(attn_bf16_kernel<8>, grid, dim3(512), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvc
