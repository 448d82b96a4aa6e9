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
//  * One workgroup = NB waves covering NB*32 query rows of one (sequence,
//    head, key split), each wave owning 32 rows.  The tile's queries sit in
//    LDS; Q fragments are re-read there every 128-key step.  Variant NB = 8 + extra block covers
//    288 rows (the 262 queries of a frame fit one workgroup): the ninth
//    32-row block is shared by waves 0..3, each taking one 32-key quarter of
//    every 128-key step, so each SIMD carries the same load (2.25 blocks);
//    their four partial softmax states are merged through LDS at the end.
//  * Keys are consumed 128 at a time (two 64-key tiles per barrier); the
//    online softmax still updates per 64-key tile.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims from LDS, B = 16 dims x
//    32 queries from registers.  In the 32x32 accumulator each lane then
//    holds 16 scores of a single query, so the row maximum and row sum are
//    in-lane reductions (shallow trees) plus one v_permlane32_swap between
//    lane l and lane l + 32.
//  * The probabilities are reused in registers as the B operand of
//    O^T = V^T P^T (A = 32 dims x 16 keys of V^T from LDS).  Which k-slot of
//    the instruction carries which key is free (k is summed over), so the
//    key order of the accumulator layout is used as is: half-wave h supplies
//    keys {4h..4h+3, 8+4h..8+4h+3} of each 16-key group.  The V pool stores
//    every 16-slot group of a V^T row in exactly that order (middle two
//    4-slot groups swapped), so a 16-byte chunk of pool memory is one MFMA
//    operand fragment.
//  * K and V^T tiles (8 KiB each) stream through a 6-stage LDS ring filled
//    by direct global->LDS loads (global_load_lds_dwordx4): up to four tiles
//    are in flight per workgroup while a pair is consumed, without staging
//    registers.  Each wave waits only for its own loads of the tile about to
//    be used (s_waitcnt vmcnt(n)) before the workgroup barrier.  16-byte
//    chunks are XOR-swizzled by row (the swizzle is applied through the
//    global addresses each lane fetches) so that fragment reads spread over
//    all LDS banks.
//  * Keys past a page's valid length: scores are set to -inf, and the V^T
//    slots of those keys are zeroed in LDS before use, so stale pool
//    contents (even NaN) never reach O.
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int D = kHeadDim;         // 64
constexpr int KT = kKeyTile;        // 64 keys per tile
constexpr int TILE_ELEMS = KT * D;  // 4096 bf16 = 8 KiB per tensor
constexpr int STAGES = 6;           // LDS ring depth in 64-key tiles (96 KiB)
constexpr int DMA_PER_TILE = 16;    // 1 KiB global->LDS loads per tile (8 for K, 8 for V)

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) with expcnt and lgkmcnt left
// open, and lgkmcnt(0) with the others left open.
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkmcnt0 = 0xC07F;
// Headroom (log2 units) the running maximum may lag the true one before the
// output accumulator is rescaled.
constexpr float kRescaleSlack = 8.f;

// 16-byte chunk c of LDS row r is stored at physical chunk c ^ swz(r).  Rows
// are 128 bytes, so 16 consecutive rows read at the same logical chunk cover
// all 64 banks exactly once, and any 8 consecutive rows cover 32 banks once.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(base + row * D + ((chunk ^ swz(row)) << 3));
}

__device__ __forceinline__ bf16x8 to_bf16x8(floatx16 s, int base) {
  floatx8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = s[base + j];
  return __builtin_convertvector(f, bf16x8);
}

// Lanes l and l+32 hold the two halves of a query's keys; these combine the
// pair with one v_permlane32_swap (which hands each lane its partner's value)
// instead of an LDS permute.  With operands (x, y) the instruction returns
// r0[l] = x[l%32] for l < 32 and y[l%32] above, r1[l] = x[32 + l%32] for
// l < 32 and y[32 + l%32] above, so for y = x, {r0, r1} is {own, partner} in
// every lane.  (The elements are copied to scalars before reinterpreting
// them: a bit cast applied directly to an element of the returned vector
// reads element 0.)
__device__ __forceinline__ void pair_values(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_values(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_values(x, a, b);
  return a + b;
}

// Maximum and sum of the 32 scores a lane holds for one 64-key tile, as
// shallow trees (depth 4-5) rather than 32-long dependency chains.
__device__ __forceinline__ float tile_max(const floatx16& a, const floatx16& b) {
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = fmaxf(fmaxf(fmaxf(a[i], a[i + 8]), b[i]), b[i + 8]);
  return fmaxf(fmaxf(fmaxf(c[0], c[1]), c[2]), fmaxf(fmaxf(fmaxf(c[3], c[4]), c[5]), fmaxf(c[6], c[7])));
}
__device__ __forceinline__ float tile_sum(const floatx16& a, const floatx16& b) {
  float u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = (a[i] + a[i + 8]) + (b[i] + b[i + 8]);
  return ((u[0] + u[1]) + (u[2] + u[3])) + ((u[4] + u[5]) + (u[6] + u[7]));
}
__device__ __forceinline__ float half_max(const floatx16& a) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fmaxf(fmaxf(a[i], a[i + 4]), fmaxf(a[i + 8], a[i + 12]));
  return fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
}
__device__ __forceinline__ float half_sum(const floatx16& a) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = (a[i] + a[i + 4]) + (a[i + 8] + a[i + 12]);
  return (c[0] + c[1]) + (c[2] + c[3]);
}

// Cursor over (table entry, 64-key tile of the page).
struct Cursor {
  int e, kt, len, pid;
};

template <class Src>
__device__ __forceinline__ void cursor_first(const Src& src, int eb, int ee, Cursor& c) {
  c.e = eb;
  c.kt = 0;
  c.len = 0;
  c.pid = 0;
  while (c.e < ee) {
    attn_entry(src, c.e, c.pid, c.len);
    if (c.len > 0) break;
    ++c.e;
  }
}

template <class Src>
__device__ __forceinline__ void cursor_next(const Src& src, int ee, Cursor& c) {
  if ((c.kt + 1) * KT < c.len) {
    ++c.kt;
    return;
  }
  c.kt = 0;
  ++c.e;
  while (c.e < ee) {
    attn_entry(src, c.e, c.pid, c.len);
    if (c.len > 0) break;
    ++c.e;
  }
}

// KV8: the pools hold FP8 (OCP E4M3) codes with per-(token, head) int8 row
// exponents (layout in kvc.h).  The ring then stages the codes and exponents
// of each tile (8,320 bytes), and after each pair's barrier the workgroup
// converts the pair into the bf16 tile layout of `lds` (two tiles), with
// v_cvt_scalef32_pk_bf16_fp8 applying 2^e; every later step is the bf16
// kernel's.  The dequantised values are exactly bf16 numbers (3-bit
// mantissas times powers of two).
template <int NB, bool XB, class Src, bool KV8 = false>
__global__ __launch_bounds__(NB * 64) void attn_bf16_kernel(const Src src) {
  static_assert(!XB || NB >= 4, "the extra block is shared by waves 0..3");
  const AttnParams& p = attn_base(src);
  constexpr int ROWS = (NB + (XB ? 1 : 0)) * 32;
  constexpr int LPT = (DMA_PER_TILE + NB - 1) / NB;  // direct loads per wave per tile
  constexpr int NBUF = KV8 ? 2 : STAGES;            // bf16 tiles: the ring, or the converted pair
  constexpr int STAGE8 = 2 * TILE_ELEMS + 2 * KT;   // FP8 stage: K codes, V codes, K exps, V exps
  __shared__ __attribute__((aligned(16))) uint16_t lds[NBUF][2][TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t lds8[KV8 ? STAGES : 1][KV8 ? STAGE8 : 16];
  __shared__ __attribute__((aligned(16))) uint16_t lds_q[ROWS * D];  // this tile's queries, swizzled rows

  // ---- which (sequence, head, split, query tile) ----------------------------
  const int L = blockIdx.x;
  const int g = L % p.groups_padded;
  const int qt = L / p.groups_padded;
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
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  // Own block: 32 rows per wave.  Extra block (XB): rows NB*32 .. NB*32+31 of
  // the tile; waves 0..3 each take one 32-key quarter of every 128-key step.
  const int wrow0 = row0 + wave * 32;
  const bool active = wrow0 < qn;
  const int qrow = wrow0 + lr;
  const bool qvalid = qrow < qn;
  const int xrow0 = row0 + NB * 32;
  const bool xblock = XB && xrow0 < qn;  // workgroup-uniform
  const bool xactive = xblock && wave < 4;
  const int xrow = xrow0 + lr;
  const bool xvalid = xblock && xrow < qn;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k_pool);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v_pool);
  const size_t page_stride = static_cast<size_t>(H) * P * D;  // elements per page (K or V)
  const size_t head_off = static_cast<size_t>(h) * P * D;

  // ---- queries of the tile -> LDS (rows past the sequence are zero) ----------
  // Q fragments (B operand of S^T = K Q^T: Q[row][16*st + 8*lh .. +7]) are read
  // from here at every 128-key step rather than held in registers.
  for (int c = tid; c < ROWS * 8; c += NB * 64) {
    const int r = c >> 3, ch = c & 7;
    const int row = row0 + r;
    i32x4 v = {0, 0, 0, 0};
    if (row < qn) v = *reinterpret_cast<const i32x4*>(qg + (static_cast<size_t>(q0 + row) * H + h) * D + ch * 8);
    *reinterpret_cast<i32x4*>(lds_q + r * D + ((ch ^ swz(r)) << 3)) = v;
  }
  // Settle the Q loads before the ring starts, so that the wait counts below
  // cover tile loads only (the first ring barrier publishes lds_q).
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

  // ---- this wave's share of each tile's 16 direct loads -----------------------
  // Load `inst` of a tile fills 1 KiB = LDS positions 64*part .. 64*part+63 of
  // K (inst < 8) or V^T (inst >= 8); lane l fills position 64*part + l, i.e.
  // row 8*part + l/8, physical chunk l%8, which holds logical chunk
  // (l%8) ^ swz(row).  Surplus slots (16 not divisible by NB) repeat the last
  // load: identical bytes to identical addresses.
  int dma_goff[LPT], dma_loff[LPT];
  bool dma_v[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int inst = min(wave * LPT + j, DMA_PER_TILE - 1);
    const int is_v = inst >> 3, part = inst & 7;
    const int row = part * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    dma_v[j] = is_v != 0;
    // K tile rows are keys ([slot][dim]); V^T tile rows are dims ([dim][slot]).
    dma_goff[j] = is_v ? row * P + chunk * 8 : row * D + chunk * 8;
    dma_loff[j] = is_v * TILE_ELEMS + part * 512;
  }
  // KV8 loads: inst 0-3 K codes (1 KiB each), 4-7 V codes, 8-11 K exponents
  // and 12-15 V exponents (16 bytes each, lane 0 only).  Stage bytes:
  // [0, 4096) K codes [slot][dim], [4096, 8192) V codes [slot][dim],
  // [8192, 8256) K exponents, [8256, 8320) V exponents.
  int dma8_kind[LPT], dma8_off[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int inst = min(wave * LPT + j, DMA_PER_TILE - 1);
    const int kind = inst >> 2, q = inst & 3;
    dma8_kind[j] = kind;
    dma8_off[j] = kind < 2 ? kind * 4096 + q * 1024 : 8192 + (kind - 2) * KT + q * 16;
  }
  const uint8_t* __restrict__ kg8 = static_cast<const uint8_t*>(p.k_pool);
  const uint8_t* __restrict__ vg8 = static_cast<const uint8_t*>(p.v_pool);
  const size_t codes_bytes = static_cast<size_t>(p.num_pool_pages) * H * P * D;  // exponents follow
  auto issue = [&](const Cursor& c, int stage) {
    if constexpr (KV8) {
      const size_t row0 = (static_cast<size_t>(c.pid) * H + h) * P + c.kt * KT;  // first slot row of the tile
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int kind = dma8_kind[j];
        const uint8_t* base = (kind & 1) ? vg8 : kg8;
        if (kind < 2) {
          // (the source goes in as const void*: a byte pointer there leaves the
          // host side of this instantiation without its launch stub)
          const void* gp = base + row0 * D + (dma8_off[j] & 4095) + lane * 16;
          __builtin_amdgcn_global_load_lds(gp, (lds_void*)(&lds8[stage][0] + dma8_off[j]), 16, 0, 0);
        } else if (lane == 0) {
          const void* gp = base + codes_bytes + row0 + (dma8_off[j] - 8192 - (kind - 2) * KT);
          __builtin_amdgcn_global_load_lds(gp, (lds_void*)(&lds8[stage][0] + dma8_off[j]), 16, 0, 0);
        }
      }
    } else {
      const size_t base = static_cast<size_t>(c.pid) * page_stride + head_off;
      const int koff = c.kt * KT * D, voff = c.kt * KT;
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const uint16_t* gp = (dma_v[j] ? vg + voff : kg + koff) + base + dma_goff[j];
        __builtin_amdgcn_global_load_lds(gp, (lds_void*)(&lds[stage][0][0] + dma_loff[j]), 16, 0, 0);
      }
    }
  };
  // KV8: converts staged tile `stage` (nk valid keys) into bf16 buffer `b`:
  // K rows keep their layout; V rows become V^T rows (dims) in the pool slot
  // order v_slot_pos with the chunk swizzle.  Keys past nk become zeros.
  auto convert = [&](int stage, int b, int nk) {
    const uint8_t* st8 = &lds8[stage][0];
    for (int it = tid; it < 2 * KT * 8; it += NB * 64) {
      const bool is_v = it >= KT * 8;
      const int r = (it >> 3) & (KT - 1), ch = it & 7;  // token, 8-dim chunk
      const uint2 w = *reinterpret_cast<const uint2*>(st8 + (is_v ? 4096 : 0) + r * D + ch * 8);
      const int e = static_cast<int8_t>(st8[8192 + (is_v ? KT : 0) + r]);
      const float sc = __builtin_ldexpf(1.f, e);
      typedef __bf16 bf16x2_ __attribute__((__vector_size__(2 * sizeof(__bf16))));
      bf16x2_ v2[4];
      v2[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.x), sc, false);
      v2[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.x), sc, true);
      v2[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.y), sc, false);
      v2[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.y), sc, true);
      uint32_t u[4];
      __builtin_memcpy(u, v2, sizeof u);
      if (r >= nk) u[0] = u[1] = u[2] = u[3] = 0u;
      if (!is_v) {
        *reinterpret_cast<uint4*>(&lds[b][0][0] + r * D + ((ch ^ swz(r)) << 3)) = make_uint4(u[0], u[1], u[2], u[3]);
      } else {
        const int pos = v_slot_pos(r);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = ch * 8 + j;  // dim
          lds[b][1][row * D + ((((pos >> 3) ^ swz(row)) << 3) | (pos & 7))] =
              static_cast<uint16_t>(u[j >> 1] >> (16 * (j & 1)));
        }
      }
    }
  };
  // Zero the V^T slots of keys nk..63 of a staged tile.  In a pool row, key k
  // of a 16-key group sits at element sigma(k) of the group (sigma swaps the
  // middle two 4-slot groups); the 16-byte chunk is then swizzled by row.
  auto zero_tail = [&](uint16_t* lv, int nk) {
    for (int it = tid; it < D * 16; it += NB * 64) {
      const int row = it >> 4, grp = it & 15;  // 4-key group in key order
      const int k0 = grp * 4;
      if (k0 + 4 <= nk) continue;
      const int sg = (grp & ~3) | ((grp & 1) << 1) | ((grp >> 1) & 1);
      const int pos = sg * 4;
      uint16_t* rp = lv + row * D + ((((pos >> 3) ^ swz(row)) << 3) | (pos & 7));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k0 + e >= nk) rp[e] = 0;
    }
  };

  float m_run = -INFINITY;  // running max of scaled scores (log2 domain)
  float l_run = 0.f;        // this lane's partial row sum
  floatx16 o0 = {}, o1 = {};
  float xm = -INFINITY, xl = 0.f;  // extra block, this wave's key quarters
  floatx16 xo0 = {}, xo1 = {};

  // Tiles are consumed two at a time (128 keys per barrier).  Tile t lives in
  // ring stage t % STAGES; up to STAGES - 2 tiles beyond the current pair are
  // in flight.
  Cursor cc, lc;
  cursor_first(src, eb, ee, cc);
  lc = cc;
  int ni = 0, nc = 0;  // tiles issued, tiles consumed
  for (int s = 0; s < STAGES - 2 && lc.e < ee; ++s) {
    issue(lc, ni % STAGES);
    cursor_next(src, ee, lc);
    ++ni;
  }
  while (nc < ni) {
    const bool two = ni >= nc + 2;
    const int outstanding = ni - nc - (two ? 2 : 1);
    if (outstanding >= 2)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LPT));
    else if (outstanding == 1)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(LPT));
    else
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __builtin_amdgcn_s_barrier();
    // The previous pair's stages are free now; they are refilled after this
    // pair's products (below), so that the waves do not all queue their loads
    // on the vector-memory pipe at the same moment.
    Cursor cb = cc;
    const int nka = min(KT, cc.len - cc.kt * KT);
    int nkb = 0;
    if (two) {
      cursor_next(src, ee, cb);
      nkb = min(KT, cb.len - cb.kt * KT);
    }
    const int sa = nc % STAGES, sb = (nc + 1) % STAGES;
    const uint16_t* lka = lds[KV8 ? 0 : sa][0];
    uint16_t* lva = lds[KV8 ? 0 : sa][1];
    const uint16_t* lkb = lds[KV8 ? 1 : sb][0];
    uint16_t* lvb = lds[KV8 ? 1 : sb][1];
    if constexpr (KV8) {
      // Everyone is done with the previous pair's bf16 tiles (barrier above).
      convert(sa, 0, nka);
      if (two) convert(sb, 1, nkb);
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
      __builtin_amdgcn_s_barrier();
    } else if (nka < KT || (two && nkb < KT)) {
      if (nka < KT) zero_tail(lva, nka);
      if (two && nkb < KT) zero_tail(lvb, nkb);
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
      __builtin_amdgcn_s_barrier();
    }

    if (active) {
      bf16x8 qf[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) qf[st] = lds_frag(lds_q, wave * 32 + lr, 2 * st + lh);
      // Operand fragments of a product group are all read from LDS before its
      // first MFMA, so the matrix pipe is not left waiting on each read.
      auto qk = [&](const uint16_t* lk, floatx16& s0, floatx16& s1) {
        bf16x8 ka[4], kb[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          ka[st] = lds_frag(lk, lr, 2 * st + lh);
          kb[st] = lds_frag(lk, 32 + lr, 2 * st + lh);
        }
        s0 = floatx16{};
        s1 = floatx16{};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], qf[st], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[st], qf[st], s1, 0, 0, 0);
        }
      };
      auto pv = [&](const floatx16& s0, const floatx16& s1, const uint16_t* lv) {
        bf16x8 va[4], vb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          va[t] = lds_frag(lv, lr, 2 * t + lh);
          vb[t] = lds_frag(lv, 32 + lr, 2 * t + lh);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 pb = to_bf16x8(t < 2 ? s0 : s1, 8 * (t & 1));
          o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], pb, o0, 0, 0, 0);
          o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[t], pb, o1, 0, 0, 0);
        }
      };
      // Softmax update of one tile's scores, in place (scores -> probabilities).
      auto soft = [&](floatx16& s0, floatx16& s1, int nk, bool full) {
        if (!full && nk < KT) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
            if (key >= nk) s0[r] = -INFINITY;
            if (key + 32 >= nk) s1[r] = -INFINITY;
          }
        }
        const float mx = pair_max(tile_max(s0, s1)) * sl2;
        // The reference maximum only moves when a row's maximum exceeds it by
        // more than kRescaleSlack (log2 units): probabilities stay <= 2^slack,
        // far from fp32 or bf16 overflow, and the final division by the row
        // sum is exact whichever reference was used.
        if (__any(mx > m_run + kRescaleSlack)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            o0[r] *= alpha;
            o1[r] *= alpha;
          }
        }
        const float nm = -m_run;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, nm));
          s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, nm));
        }
        l_run += tile_sum(s0, s1);
      };
      floatx16 a0, a1, b0, b1;
      if (two && nka == KT && nkb == KT) {
        // Full pair: one straight-line block with a single softmax update for
        // all 128 keys.  Waves w and w+4 share a SIMD; the upper half takes the
        // pair in the opposite order so that one wave's softmax arithmetic
        // tends to run under the other's products.
        const bool rev = (wave & 4) != 0;
        const uint16_t* k1 = rev ? lkb : lka;
        const uint16_t* k2 = rev ? lka : lkb;
        const uint16_t* v1 = rev ? lvb : lva;
        const uint16_t* v2 = rev ? lva : lvb;
        __builtin_amdgcn_s_setprio(1);
        qk(k1, a0, a1);
        qk(k2, b0, b1);
        __builtin_amdgcn_s_setprio(0);
        const float mx = pair_max(fmaxf(tile_max(a0, a1), tile_max(b0, b1))) * sl2;
        if (__any(mx > m_run + kRescaleSlack)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            o0[r] *= alpha;
            o1[r] *= alpha;
          }
        }
        const float nm = -m_run;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          a0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(a0[r], sl2, nm));
          a1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(a1[r], sl2, nm));
          b0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(b0[r], sl2, nm));
          b1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(b1[r], sl2, nm));
        }
        l_run += tile_sum(a0, a1) + tile_sum(b0, b1);
        pv(a0, a1, v1);
        pv(b0, b1, v2);
      } else {
        qk(lka, a0, a1);
        soft(a0, a1, nka, false);
        pv(a0, a1, lva);
        if (two) {
          qk(lkb, b0, b1);
          soft(b0, b1, nkb, false);
          pv(b0, b1, lvb);
        }
      }
    }

    if (XB && xactive) {
      // Extra block: this wave's 32-key quarter of the 128-key step.
      const int tile = wave >> 1, kb = wave & 1;
      const int nkt = tile ? (two ? nkb : 0) : nka;
      if (nkt > 32 * kb) {
        const uint16_t* lk = tile ? lkb : lka;
        const uint16_t* lv = tile ? lvb : lva;
        floatx16 s = {};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 4; ++st)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_frag(lk, 32 * kb + lr, 2 * st + lh),
                                                      lds_frag(lds_q, NB * 32 + lr, 2 * st + lh), s, 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
        if (nkt < 32 * kb + 32) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * kb + (r >> 2) * 8 + lh * 4 + (r & 3);
            if (key >= nkt) s[r] = -INFINITY;
          }
        }
        const float mx = pair_max(half_max(s)) * sl2;
        if (__any(mx > xm + kRescaleSlack)) {
          const float m_new = fmaxf(xm, mx);
          const float alpha = __builtin_amdgcn_exp2f(xm - m_new);
          xm = m_new;
          xl *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            xo0[r] *= alpha;
            xo1[r] *= alpha;
          }
        }
        const float nm = -xm;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, nm));
        xl += half_sum(s);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 pb = to_bf16x8(s, 8 * ks);
          const int ch = 2 * (2 * kb + ks) + lh;
          xo0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_frag(lv, lr, ch), pb, xo0, 0, 0, 0);
          xo1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_frag(lv, 32 + lr, ch), pb, xo1, 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    for (int s = 0; s < 2 && lc.e < ee; ++s) {
      issue(lc, ni % STAGES);
      cursor_next(src, ee, lc);
      ++ni;
    }
    nc += two ? 2 : 1;
    if (two) cc = cb;
    cursor_next(src, ee, cc);
  }

  // ---- epilogue ---------------------------------------------------------------
  // Writes one 32-row block: normalised O (bf16) and lse, or the split's
  // partial O (fp32) and lse.  m is the running maximum, ltot the row sum.
  auto write_block = [&](int row, bool valid, const floatx16& a0, const floatx16& a1, float m, float ltot) {
    const bool empty = !(ltot > 0.f);
    const float inv = empty ? 0.f : 1.f / ltot;
    const float lse_nat = empty ? -INFINITY : (m + __log2f(ltot)) * 0.69314718055994530942f;
    if (!valid) return;
    const size_t orow = static_cast<size_t>(q0 + row) * H + h;
    if (p.num_splits == 1) {
      uint16_t* og = static_cast<uint16_t*>(p.o) + orow * D;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          floatx4 f;
#pragma unroll
          for (int j = 0; j < 4; ++j) f[j] = (db ? a1 : a0)[r4 * 4 + j] * inv;
          *reinterpret_cast<bf16x4*>(og + db * 32 + r4 * 8 + lh * 4) = __builtin_convertvector(f, bf16x4);
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
          for (int j = 0; j < 4; ++j) f[j] = (db ? a1 : a0)[r4 * 4 + j] * inv;
          *reinterpret_cast<floatx4*>(po + db * 32 + r4 * 8 + lh * 4) = f;
        }
      }
      if (lh == 0) p.part_lse[static_cast<size_t>(split) * p.total_q * H + orow] = lse_nat;
    }
  };

  if (XB && xblock) {
    // Combine the extra block's four key-quarter states: waves 1..3 hand
    // theirs to wave 0 through LDS (the ring is idle: every issued tile has
    // been consumed, and the barrier below orders the reuse).
    float* xbuf = reinterpret_cast<float*>(&lds[0][0][0]);  // [3][64 dims][32 rows]
    float* xms = xbuf + 3 * 64 * 32;                        // [3][32]
    float* xls = xms + 3 * 32;                              // [3][32]
    const float xl_tot = pair_sum(xl);
    __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    __builtin_amdgcn_s_barrier();
    if (wave >= 1 && wave < 4) {
      float* b = xbuf + (wave - 1) * 64 * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = (r >> 2) * 8 + lh * 4 + (r & 3);
        b[d * 32 + lr] = xo0[r];
        b[(32 + d) * 32 + lr] = xo1[r];
      }
      if (lh == 0) {
        xms[(wave - 1) * 32 + lr] = xm;
        xls[(wave - 1) * 32 + lr] = xl_tot;
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    __builtin_amdgcn_s_barrier();
    if (wave == 0) {
      float mw[3], lw[3];
      float M = xm;
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        mw[w] = xms[w * 32 + lr];
        lw[w] = xls[w * 32 + lr];
        M = fmaxf(M, mw[w]);
      }
      const float c0 = xm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(xm - M);
      float cw[3];
      float Lt = xl_tot * c0;
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        cw[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        Lt += lw[w] * cw[w];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = (r >> 2) * 8 + lh * 4 + (r & 3);
        float a = xo0[r] * c0, b = xo1[r] * c0;
#pragma unroll
        for (int w = 0; w < 3; ++w) {
          a = __builtin_fmaf(xbuf[(w * 64 + d) * 32 + lr], cw[w], a);
          b = __builtin_fmaf(xbuf[(w * 64 + 32 + d) * 32 + lr], cw[w], b);
        }
        xo0[r] = a;
        xo1[r] = b;
      }
      write_block(xrow, xvalid, xo0, xo1, M, Lt);
    }
  }
  if (!active) return;
  const float l_tot = pair_sum(l_run);
  write_block(qrow, qvalid, o0, o1, m_run, l_tot);
}

}  // namespace

// waves <= 8: that many 32-row blocks; 9: eight waves plus the shared extra block.
int attn_bf16_rows_per_tile(int waves) { return waves * 32; }

template <bool KV8, class Src>
static hipError_t launch_impl(const Src& src, int waves, hipStream_t stream) {
  const AttnParams& p = attn_base(src);
  const dim3 grid(static_cast<unsigned>(p.q_tiles) * p.groups_padded);
  switch (waves) {
#define KVC_CASE(W)                                                                                    \
  case W:                                                                                              \
    hipLaunchKernelGGL((attn_bf16_kernel<W, false, Src, KV8>), grid, dim3(W * 64), 0, stream, src); \
    break;
    KVC_CASE(1)
    KVC_CASE(2)
    KVC_CASE(3)
    KVC_CASE(4)
    KVC_CASE(5)
    KVC_CASE(6)
    KVC_CASE(7)
    KVC_CASE(8)
#undef KVC_CASE
    case 9:
      hipLaunchKernelGGL((attn_bf16_kernel<8, true, Src, KV8>), grid, dim3(8 * 64), 0, stream, src);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream) {
  return launch_impl<false>(p, waves, stream);
}
hipError_t launch_attn_bf16(const AttnParamsInline& p, int waves, hipStream_t stream) {
  return launch_impl<false>(p, waves, stream);
}
hipError_t launch_attn_fp8kv(const AttnParams& p, int waves, hipStream_t stream) {
  return launch_impl<true>(p, waves, stream);
}
hipError_t launch_attn_fp8kv(const AttnParamsInline& p, int waves, hipStream_t stream) {
  return launch_impl<true>(p, waves, stream);
}

}  // namespace kvc
