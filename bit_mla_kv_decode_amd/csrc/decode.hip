// Split-KV decode attention over the paged low-bit MLA cache (gfx950).
//
// Math (absorbed MLA decode; QuantMLA's low-bit kernel unpacks and
// dequantizes the cache inside attention -- "QuantMLA: INT4 (and INT2) for
// both halves of the MLA cache", flowchart and Key findings, systems):
//   S[h, t] = scale * <q[h, 0:576], khat[t, 0:576]>       (latent + RoPE key)
//   O[h, :] = sum_t softmax_t(S[h, :]) * khat[t, 0:512]   (latent is the value)
//
// One workgroup = one piece of work (a page range of one sequence: a fixed
// split, or a share of the balanced partition), 256 threads = 4 wavefronts,
// one per SIMD.  Wave w owns heads [32w, 32w + 32); at 17..64 rows per
// sequence the wavefronts of a head group split its channels instead (four
// per group at 17..32 rows, two workgroups per compute unit; two per group at
// 33..64 rows), sharing one softmax through LDS, see split_pass_cs; at <= 16
// rows (quantized formats) the four wavefronts work independently, each on
// its own 32-token tiles, see process_range_iw.  The work
// is tiled by half pages (32 tokens):
//   1. fill: every thread loads its share of the next tile's packed bytes
//      (16-byte loads; the 32 lanes of a half-wave read 512 contiguous bytes of
//      one code chunk), dequantizes them in registers once for all heads
//      (bf16(fma(code, S, Z))) and writes a bf16 tile khat[32][576] to LDS
//      (rows padded to 1168 bytes).  Tiles are double buffered, so the loads
//      of tile k+1 are in flight while tile k computes.
//   2. Q.K^T on MFMA 32x32x16 bf16: A = khat rows (ds_read_b128), B = q^T
//      (half of the k-steps staged in LDS, half in registers), giving
//      S^T[token][head]: each lane holds one head and 16 tokens per block.
//   3. softmax weights in registers: per-head max over the lane's tokens, the
//      other half-wave via v_permlane32_swap; exp2 with the scale folded into
//      log2 units.  Weights are taken against a fixed reference per piece (the
//      first tile's max, lifted), so O is never rescaled and stays in the MFMA
//      accumulators; a piece whose logits rise beyond the reference's range
//      is recomputed with its true max (see split_pass).
//   4. P.V on MFMA 32x32x16 bf16 with the latent as value: A = khat^T read
//      with ds_read_b64_tr_b16 (transposing 16-bit loads) from the same tile,
//      B = P straight from the softmax registers (through LDS where the
//      channels are split).  P is split into a bf16 high
//      part and a bf16 remainder (two MFMAs sharing A) so the weights keep
//      ~16 significant bits; a single bf16 P loses too much accuracy when a few
//      tokens with large, cancelling latent values dominate a head.
//      O^T[channel][head] accumulates in 256 fp32 registers per lane.
//   5. per piece: O / l and lse = m + log l are written as fp32 partials (or,
//      with one split, the final bf16 output directly).
// A second kernel merges the pieces with log-sum-exp weights.
#include <atomic>
#include <type_traits>

#include "append.h"
#include "kernels.h"

namespace mla {

constexpr int kTileTok = 32;                // tokens per tile (half a page)
constexpr int kRow = kD + 8;                // LDS row stride in bf16: 1168 B
constexpr int kTile = kTileTok * kRow;      // elements per tile buffer (37376 bytes)
// q of all heads is split between LDS and registers by k-step (16 channels):
// the even k-steps 0, 2, .., 30 (256 channels) are staged in LDS (rows padded
// to 528 bytes so 16 heads reading the same chunk hit distinct banks), the
// odd k-steps 1, .., 31 and 32..35 stay in registers.  Interleaving keeps the
// Q.K^T loop at no more than two LDS operand reads per MFMA pair, and the
// register share keeps the hot loop free of spills.
constexpr int kQLds = 256;
constexpr int kQRow = kQLds + 8;
constexpr int kQRegSteps = (kD - kQLds) / 16;   // 20 k-steps of 16 channels in registers
__device__ __forceinline__ constexpr bool q_in_lds(int ks) { return ks < 32 && (ks & 1) == 0; }
__device__ __forceinline__ constexpr int q_reg_index(int ks) { return ks < 32 ? ks >> 1 : ks - 16; }
constexpr int kThreads = 256;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS tile: 32 rows of 1168 bytes (576 bf16 + 16 bytes of padding); token t
// of the tile lives in row rho(t), which transposes every 4 x 4 block of
// tokens inside a group of 16: rho(16u + 4q + j) = 16u + 4j + q.  Chunk c
// (channels 8c .. 8c + 7) of a row is at byte 16 c.  With 1168 = 144 (mod 256):
//  - 16 consecutive rows read at the same chunk (Q.K^T operand reads, one
//    16-lane pass of ds_read_b128) fall in 16 distinct 16-byte bank groups;
//  - the 4 tokens a transposing read gathers (4q' + j, j < 4) sit in rows
//    4 apart, i.e. in 4 distinct 64-byte bank blocks, so the 32 lanes of a
//    pass (4 rows x 64 bytes) are conflict-free as well.
// All addresses stay affine in the unrolled loop indices.
__device__ __forceinline__ int rho(int t) { return (t & ~15) + 4 * (t & 3) + ((t >> 2) & 3); }
__device__ __forceinline__ int tile_off(int r, int chunk) { return r * kRow + 8 * chunk; }

__device__ __forceinline__ float wave_partner(float v) {
  // value of lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                            false, false);
  const unsigned other = (threadIdx.x & 32) ? r[0] : r[1];
  return __builtin_bit_cast(float, other);
}

// Q.K^T logits accumulated in VGPRs.  Beside the 256 O accumulators of the
// > 64-row kernel (all AGPRs) the compiler gives a builtin MFMA chain an AGPR
// destination as well and swaps one O block through VGPRs around every tile
// (48 accumulator moves per tile, plus 16 more to read the logits out).
// Written as inline asm with VGPR operands the chain needs none.  The compiler
// does not see the matrix-pipe hazards of asm, so each MFMA is issued two wait
// states after whatever precedes it (a VALU write of an operand needs them) and
// the chain ends with 24 wait states, more than a 32x32 MFMA needs before a
// VALU instruction reads or overwrites its result; a dependent MFMA reading
// the previous one's result as its accumulator may follow at once.
__device__ __forceinline__ void mfma_v_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_drain(f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d));
}

// ---------------------------------------------------------------- dequantization

// w & m, opaque to the optimizer: keeps one AND per masked word (a plain &
// lets the compiler rewrite the mask-and-convert sequence into more
// instructions).
__device__ __forceinline__ unsigned mask_bytes(unsigned w, unsigned m) {
  unsigned r;
  asm volatile("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(w), "v"(m));
  return r;
}

using h2 = _Float16 __attribute__((ext_vector_type(2)));

// Codes with no conversion instruction at all: a code c alone in bits
// [k, k + b) of a 16-bit half (k + b <= 10, the other bits zero) is the fp16
// subnormal c 2^(k - 24), exact.  v_fma_mix_f32 takes it as one operand, S
// 2^(24 - k) in fp32 as the other (exact: S has 11 significant bits) and Z
// from the packed pair: the product is c S exactly and the sum is rounded
// once, i.e. fma(code, S, Z) in fp32.  SzScaled<N> holds S 2^(24 - k) for the
// N bit offsets k = 0, b, 2b, .. a format uses (4-bit codes at k = 0, 4;
// 2-bit codes at k = 0, 2, 4, 6) and the pair, whose Z half is read as is.
template <int N> struct SzScaled {
  float s[N];
  unsigned sz;
};
template <int N, int kBits>
__device__ __forceinline__ SzScaled<N> sz_scaled(unsigned sz) {
  const _Float16 S = __builtin_bit_cast(h2, sz)[0];
  SzScaled<N> r;
  // one v_fma_mix_f32 each (S >= 0, so adding +0 changes nothing)
#pragma unroll
  for (int i = 0; i < N; ++i) r.s[i] = __builtin_fmaf((float)S, (float)(1 << (24 - kBits * i)), 0.0f);
  r.sz = sz;
  return r;
}
__device__ __forceinline__ float dq_sub(_Float16 c, float s, unsigned sz) {
  return __builtin_fmaf((float)c, s, (float)__builtin_bit_cast(h2, sz)[1]);
}
__device__ __forceinline__ h2 as_h2(unsigned w) { return __builtin_bit_cast(h2, w); }

// 2-bit codes: element e of a dword sits at bit 2 e; m[j] (j < 4) keeps
// elements j and j + 8 in place (bits 2 j and 16 + 2 j), m[j] (j >= 4) the
// same of the dword shifted right by 8.  Half hf of m[j] gives element 8 hf +
// j, against scale j % 4 (2^(24 - 2 (j % 4)) S).
__device__ __forceinline__ void int2_split(unsigned w, unsigned (&m)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = mask_bytes(w, 0x00030003u << (2 * j));
  const unsigned w8 = w >> 8;
#pragma unroll
  for (int j = 4; j < 8; ++j) m[j] = mask_bytes(w8, 0x00030003u << (2 * (j - 4)));
}

// ---------------------------------------------------------------- tile fills
// A tile is half a page: tokens [32 hp, 32 hp + 32) of one physical page.
// Thread mapping: lane l = tid % 32 takes token t = rho(l) and cs = tid / 32
// selects chunks.  The 32 lanes of a half-wave still read 512 contiguous bytes
// of one code chunk (rho permutes the tokens among them), and since rho is its
// own inverse the token's tile row rho(t) is l: the lanes of a 16-byte tile
// write hit consecutive rows, which spread over the LDS banks without
// conflicts, where writing rows rho(l) cost 8 conflict cycles per write.
// load(page, hp): issue this thread's global loads into registers.
// store(tile, nvalid): dequantize into the LDS tile; rows >= nvalid are zero.

template <int F> struct Fill;

// Every thread also dequantizes 8 RoPE channels of its token: channels
// [8 cs, 8 cs + 8), i.e. dword cs % 4 of RoPE chunk cs / 4.
// The dequantization of a tile is split into kSubsteps small steps (one packed
// pair of bf16 values each, a 16-byte LDS write every 4 steps) so the kernel
// can place one step after each P.V MFMA of the previous tile.

template <> struct Fill<kC4R4> {
  using Lay = PageLayout<kC4R4>;
  static constexpr int kSubsteps = 36;  // 9 dwords (8 content + 1 RoPE) x 4 pairs
  u32x4 c[2];
  unsigned sz[2];
  unsigned r, rsz;
  bool ok;
  // working state of the dword being converted: its elements split as
  // dq_int4x8 does, and the (S, Z) of its group (see SzScaled)
  unsigned ma, mb, mc, md, outw[4];
  SzScaled<2> zs;
  const uint8_t* base;  // page of the pending tile
  int hp;               // its half of the page
  static constexpr int kLoads = 6;
  __device__ __forceinline__ void begin(const uint8_t* __restrict__ cache, int64_t page, int half, int64_t num_pages) {
    ok = page >= 0 && page < num_pages;
    base = cache + (ok ? page : 0) * (int64_t)Lay::kBytes;  // an invalid page reads page 0, zeroed at store
    hp = half;
  }
  // load i of the tile: content chunks cs and cs + 8 (channels [32 j, 32 j + 32),
  // group j / 2) with their scale/zero, then the RoPE dword and its scale/zero
  __device__ __forceinline__ void issue(int i) {
    const int t = rho(threadIdx.x & 31) + 32 * hp, cs = threadIdx.x >> 5;
    const int j = cs + 8 * (i >> 1);
    if (i == 0 || i == 2) c[i >> 1] = *(const u32x4*)(base + Lay::kCodesA + (j * kPage + t) * 16);
    if (i == 1 || i == 3) sz[i >> 1] = *(const unsigned*)(base + Lay::kSzB + ((j >> 1) * kPage + t) * 4);
    if (i == 4) r = *(const unsigned*)(base + Lay::kCodesC + ((cs >> 2) * kPage + t) * 16 + 4 * (cs & 3));
    if (i == 5) rsz = *(const unsigned*)(base + Lay::kSzD + t * 4);
  }
  __device__ __forceinline__ void load(const uint8_t* __restrict__ cache, int64_t page, int half, int64_t num_pages) {
    begin(cache, page, half, num_pages);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) issue(i);
  }
  // step u: dword p = u / 4 (p < 8: content chunk cs + 8 (p / 4), dword p % 4;
  // p = 8: RoPE), pair q = u % 4 (elements 2q, 2q + 1 of the dword)
  __device__ __forceinline__ void substep(__bf16* tile, int nvalid, int u) {
    const int l = threadIdx.x & 31, t = rho(l), cs = threadIdx.x >> 5;  // token rho(l) lives in row l
    const int p = u >> 2, q = u & 3;
    if (q == 0) {
      if ((p & 3) == 0) {  // a new group: content dwords 0 and 4, the RoPE dword
        const bool live = ok && t < nvalid;  // dead rows: S = Z = 0 gives exact zeros
        zs = sz_scaled<2, 4>(live ? (p < 8 ? sz[p >> 2] : rsz) : 0u);
      }
      const unsigned w = p < 8 ? c[p >> 2][p & 3] : r;
      ma = mask_bytes(w, 0x000F000Fu);        // elements 0, 4 (2^24 S)
      mb = mask_bytes(w, 0x00F000F0u);        // elements 1, 5 (2^20 S)
      mc = mask_bytes(w >> 8, 0x000F000Fu);   // elements 2, 6
      md = mask_bytes(w >> 8, 0x00F000F0u);   // elements 3, 7
    }
    // pair q: elements 2q, 2q + 1 = half q / 2 of (ma, mb) (q even) or (mc, md)
    const int hf = q >> 1;
    const float a = dq_sub(as_h2((q & 1) ? mc : ma)[hf], zs.s[0], zs.sz);
    const float b = dq_sub(as_h2((q & 1) ? md : mb)[hf], zs.s[1], zs.sz);
    outw[q] = pack_bf16x2(a, b);
    if (q == 3) {
      const int chunk = p < 8 ? 4 * (cs + 8 * (p >> 2)) + (p & 3) : 64 + cs;
      *(u32x4*)(tile + l * kRow + 8 * chunk) = (u32x4){outw[0], outw[1], outw[2], outw[3]};
    }
  }
  __device__ __forceinline__ void store(__bf16* tile, int nvalid) {
#pragma unroll
    for (int u = 0; u < kSubsteps; ++u) substep(tile, nvalid, u);
  }
};

template <> struct Fill<kC2R4> {
  using Lay = PageLayout<kC2R4>;
  static constexpr int kSubsteps = 36;  // 4 content dwords x 8 pairs + 1 RoPE dword x 4 pairs
  u32x4 c;
  unsigned sz[2];
  unsigned r, rsz;
  bool ok;
  unsigned ma, mb, mc, md, outl[4], outh[4];  // masked words; packed pairs of both halves
  SzScaled<4> zs;  // (S, Z) of the group: 2^24 S, 2^22 S, 2^20 S, 2^18 S (RoPE: s[0], s[2])
  const uint8_t* base;  // page of the pending tile
  int hp;               // its half of the page
  static constexpr int kLoads = 5;
  __device__ __forceinline__ void begin(const uint8_t* __restrict__ cache, int64_t page, int half, int64_t num_pages) {
    ok = page >= 0 && page < num_pages;
    base = cache + (ok ? page : 0) * (int64_t)Lay::kBytes;  // an invalid page reads page 0, zeroed at store
    hp = half;
  }
  // load i of the tile: content chunk cs = channels [64 cs, 64 cs + 64) = groups
  // 2 cs, 2 cs + 1, their two scale/zero pairs, the RoPE dword and its scale/zero
  __device__ __forceinline__ void issue(int i) {
    const int t = rho(threadIdx.x & 31) + 32 * hp, cs = threadIdx.x >> 5;
    if (i == 0) c = *(const u32x4*)(base + Lay::kCodesA + (cs * kPage + t) * 16);
    if (i == 1 || i == 2) sz[i - 1] = *(const unsigned*)(base + Lay::kSzB + ((2 * cs + i - 1) * kPage + t) * 4);
    if (i == 3) r = *(const unsigned*)(base + Lay::kCodesC + ((cs >> 2) * kPage + t) * 16 + 4 * (cs & 3));
    if (i == 4) rsz = *(const unsigned*)(base + Lay::kSzD + t * 4);
  }
  __device__ __forceinline__ void load(const uint8_t* __restrict__ cache, int64_t page, int half, int64_t num_pages) {
    begin(cache, page, half, num_pages);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) issue(i);
  }
  // steps 0..31: content dword v = u / 8 (channels [64 cs + 16 v, +16), group
  // 2 cs + v / 2), pair q = u % 8 (elements 2q, 2q + 1); steps 32..35: RoPE
  __device__ __forceinline__ void substep(__bf16* tile, int nvalid, int u) {
    const int l = threadIdx.x & 31, t = rho(l), cs = threadIdx.x >> 5;  // token rho(l) lives in row l
    const bool live = ok && t < nvalid;  // dead rows: S = Z = 0 gives exact zeros
    __bf16* row = tile + l * kRow;
    if (u < 32) {
      // step 2 i + h of dword v: elements 2i, 2i + 1 (h = 0) or 8 + 2i, 8 + 2i + 1
      // (h = 1), the low and high halves of the same two masked words: element
      // j < 4 of a half sits at bit 2 j of the dword, element j >= 4 at bit
      // 2 (j - 4) of the dword shifted by 8 (scale j % 4)
      const int v = u >> 3, i = (u & 7) >> 1, h = u & 1;
      if (h == 0) {
        if ((u & 7) == 0 && (v & 1) == 0) zs = sz_scaled<4, 2>(live ? sz[v >> 1] : 0u);
        const unsigned w = i < 2 ? c[v] : c[v] >> 8;
        ma = mask_bytes(w, 0x00030003u << (2 * ((2 * i) & 3)));
        mb = mask_bytes(w, 0x00030003u << (2 * ((2 * i + 1) & 3)));
      }
      const float ea = dq_sub(as_h2(ma)[h], zs.s[(2 * i) & 3], zs.sz);
      const float eb = dq_sub(as_h2(mb)[h], zs.s[(2 * i + 1) & 3], zs.sz);
      (h ? outh : outl)[i] = pack_bf16x2(ea, eb);
      if ((u & 7) == 7) {
        *(u32x4*)(row + 8 * (8 * cs + 2 * v)) = (u32x4){outl[0], outl[1], outl[2], outl[3]};
        *(u32x4*)(row + 8 * (8 * cs + 2 * v + 1)) = (u32x4){outh[0], outh[1], outh[2], outh[3]};
      }
    } else {
      // RoPE dword, 4-bit codes, split as dq_int4x8 does: pair q = elements
      // 2q, 2q + 1 = half q / 2 of (ma, mb) (q even) or (mc, md)
      const int q = u - 32, hf = q >> 1;
      if (q == 0) {
        zs = sz_scaled<4, 2>(live ? rsz : 0u);
        ma = mask_bytes(r, 0x000F000Fu);
        mb = mask_bytes(r, 0x00F000F0u);
        mc = mask_bytes(r >> 8, 0x000F000Fu);
        md = mask_bytes(r >> 8, 0x00F000F0u);
      }
      const float ea = dq_sub(as_h2((q & 1) ? mc : ma)[hf], zs.s[0], zs.sz);
      const float eb = dq_sub(as_h2((q & 1) ? md : mb)[hf], zs.s[2], zs.sz);
      outl[q] = pack_bf16x2(ea, eb);
      if (q == 3) *(u32x4*)(row + 8 * (64 + cs)) = (u32x4){outl[0], outl[1], outl[2], outl[3]};
    }
  }
  __device__ __forceinline__ void store(__bf16* tile, int nvalid) {
#pragma unroll
    for (int u = 0; u < kSubsteps; ++u) substep(tile, nvalid, u);
  }
};

// Unquantized baseline: 32 rows x 72 chunks of 16 bytes, copied through
// registers (nine chunks per thread, in three rounds) at store time.  Rows of
// the page past the sequence end are read (they are inside the page) and
// replaced by zeros.
template <> struct Fill<kBF16> {
  static constexpr int kSubsteps = 0;
  static constexpr int kLoads = 0;
  const uint8_t* base;
  bool ok;
  __device__ __forceinline__ void substep(__bf16*, int, int) {}
  __device__ __forceinline__ void begin(const uint8_t* __restrict__ cache, int64_t page, int hp, int64_t num_pages) {
    ok = page >= 0 && page < num_pages;
    base = cache + (ok ? page : 0) * (int64_t)PageLayout<kBF16>::kBytes + hp * (kTileTok * kD * 2);
  }
  __device__ __forceinline__ void issue(int) {}
  __device__ __forceinline__ void load(const uint8_t* __restrict__ cache, int64_t page, int hp, int64_t num_pages) {
    begin(cache, page, hp, num_pages);
  }
  __device__ __forceinline__ void store(__bf16* tile, int nvalid) const {
#pragma unroll
    for (int round = 0; round < 3; ++round) {
      u32x4 v[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) v[i] = *(const u32x4*)(base + (threadIdx.x + kThreads * (3 * round + i)) * 16);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int ci = threadIdx.x + kThreads * (3 * round + i);  // 0 .. 2303
        const int t = ci / 72, col = ci % 72;
        const bool live = ok && t < nvalid;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *(u32x4*)(tile + tile_off(rho(t), col)) = live ? v[i] : z;
      }
    }
  }
};

// ---------------------------------------------------------------- decode kernel

// Block-table window for the tiles [k0, k1) of a split: lane i holds the id of
// page wbase + i, so the page of a tile comes from v_readlane without a
// memory wait; the window moves every 64 pages.
struct PageWindow {
  const int32_t* bt;
  int p_end, wbase, ids;
  __device__ __forceinline__ PageWindow(const int32_t* bt_, int k0, int k1) : bt(bt_) {
    p_end = (k1 + 1) >> 1;
    wbase = k0 >> 1;
    const int lane = threadIdx.x & 63;
    ids = wbase + lane < p_end ? bt[wbase + lane] : -1;
  }
  // The lane read sits in both branches, so the wait for a window load stays
  // on the (rare) refill path instead of draining every load in flight.
  __device__ __forceinline__ int page_of(int kt) {
    const int pg = kt >> 1;
    if (pg - wbase >= 64) {  // uniform; once per 64 pages
      wbase = pg;
      const int lane = threadIdx.x & 63;
      ids = wbase + lane < p_end ? bt[wbase + lane] : -1;
      return __builtin_amdgcn_readlane(ids, 0);
    }
    return __builtin_amdgcn_readlane(ids, pg - wbase);
  }
};

// Result of one pass over a split, per lane: O^T accumulators (channels x the
// lane's head), softmax denominator part and reference.
struct SplitAcc {
  f32x16 o[16];
  float l_sum;   // this lane's share of sum_t p_t
  float m_ref;   // reference (log2 units) the p_t are taken against
  float m_seen;  // true max logit of the head over the split (log2 units)
};

// Softmax weights are taken against a fixed reference per split, so O never
// needs rescaling and stays in MFMA accumulators.  The reference is the first
// tile's max plus kRefLift (log2 units): weights of tokens more than
// 126 - kRefLift below that max flush to zero (they are below 2^-86 of the
// largest weight), and later tiles may rise up to kRefLift + kMaxLift above
// it with p <= 2^kMaxLift, which keeps l and O below 2^113 even for 2^17
// tokens of magnitude 2^16.  If any logit of the split lies more than
// kMaxLift above the reference, the pass reports it and the caller recomputes
// the split with the reference set to the split's true max.
constexpr float kRefLift = 40.0f;
constexpr float kMaxLift = 80.0f;

// Rows.  With s_q query tokens per sequence and H heads, the rows of sequence
// b are (query i, head h) -> i H + h, which is how q, the outputs and the
// partial rows are laid out.  Head chunk c of a launch covers heads
// [c Hc, c Hc + Hc) of every query: workgroup row r -> (r / Hc, c Hc + r % Hc).
// Query i sees tokens [0, L - (s_q - 1) + i) (the query tokens are the last
// s_q of the sequence, each seeing itself and the ones before it).
struct RowOf {
  int g;      // row of the sequence
  int limit;  // tokens visible to it
  bool valid;
};

__device__ __forceinline__ RowOf row_of(const DecodeArgs& a, int chunk, int L, int r) {
  const int i = r / a.chunk_heads, h = chunk * a.chunk_heads + r % a.chunk_heads;
  RowOf o;
  o.valid = i < a.s_q && h < a.qheads;
  o.g = i * a.qheads + h;
  o.limit = L - (a.s_q - 1) + i;
  return o;
}

// A reference that stays finite when a row sees no token of the piece (its
// logits are all -inf): the weights are then exactly 0.
__device__ __forceinline__ float finite_ref(float m) { return fmaxf(m, -3.0e38f); }

template <int F>
__device__ __forceinline__ bool split_pass(const DecodeArgs& a, __bf16* smem, const int32_t* bt, int L, int k0,
                                           int k1, const bf16x8 (&qr)[kQRegSteps], int limit, bool fixed,
                                           float m_fixed, SplitAcc& acc) {
  const int limit_min = L - (a.s_q - 1);  // the smallest row limit (uniform)
  const int lane = threadIdx.x & 63, hi = lane >> 5;
  const __bf16* qrow = smem + 2 * kTile + ((threadIdx.x >> 6) * 32 + (lane & 31)) * kQRow + 8 * hi;
  // transposing-read addresses for the P.V operand: lane (g, i) = (lane / 16,
  // lane % 16) reads 4 channels of one token row; see the kernel comment.
  const int g = lane >> 4, i16 = lane & 15;
  // token 4 quad + i16 / 4 of a 16-token step sits in row 4 (i16 / 4) + quad;
  // quad = g / 2 for the first 4 k-slots of the lane, 2 + g / 2 for the next 4
  const int tr_row0 = 4 * (i16 >> 2) + (g >> 1);
  const int tr_chunk = 2 * (g & 1) + ((i16 & 3) >> 1);   // + 4 ct
  const int tr_half = 4 * (i16 & 1);

#pragma unroll
  for (int ct = 0; ct < 16; ++ct) acc.o[ct] = (f32x16){};
  acc.l_sum = 0.0f;
  acc.m_ref = fixed ? finite_ref(m_fixed) : -INFINITY;
  acc.m_seen = -INFINITY;
  bool lifted = false;

  PageWindow win(bt, k0, k1);

  Fill<F> fill;
  fill.load(a.cache, win.page_of(k0), k0 & 1, a.num_pages);
  fill.store(smem, min(kTileTok, L - k0 * kTileTok));
  __syncthreads();

  for (int k = k0; k < k1; ++k) {
    __bf16* tile = smem + ((k - k0) & 1) * kTile;
    __bf16* next = smem + ((k - k0 + 1) & 1) * kTile;
    // next tile's loads (the last iteration reloads its own tile: harmless,
    // keeps the loop body a single basic block so VALU and MFMA interleave),
    // issued one every kLoadEvery k-steps of Q.K^T below: a burst of them
    // would hold the wavefront's in-order issue while the memory pipeline
    // takes them, with no MFMA running alongside
    const int kn = min(k + 1, k1 - 1);
    fill.begin(a.cache, win.page_of(kn), kn & 1, a.num_pages);
    constexpr int kLoadEvery = 3;

    // ---- S^T = khat . q^T for the 32 tokens of the tile (in VGPRs, see
    //      mfma_v_first).  Operands are read 4 k-steps ahead; scheduling
    //      barriers pin that order so LDS latency hides behind the MFMAs
    //      instead of stalling each one.
    f32x16 s;
    const __bf16* arow = tile + rho(lane & 31) * kRow + 8 * hi;
    bf16x8 kv[4], qv[2];
#pragma unroll
    for (int d = 0; d < 4; ++d) kv[d] = *(const bf16x8*)(arow + 16 * d);
#pragma unroll
    for (int d = 0; d < 2; ++d) qv[d] = *(const bf16x8*)(qrow + 16 * d);   // k-steps 0, 2
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 bq = q_in_lds(ks) ? qv[(ks >> 1) & 1] : qr[q_in_lds(ks) ? 0 : q_reg_index(ks)];
      if (ks == 0)
        mfma_v_first(s, kv[0], bq);
      else
        mfma_v_acc(s, kv[ks & 3], bq);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 4 < 36) kv[ks & 3] = *(const bf16x8*)(arow + 16 * (ks + 4));
      if (q_in_lds(ks) && ks + 4 < 32) qv[(ks >> 1) & 1] = *(const bf16x8*)(qrow + 16 * ((ks >> 1) + 2));
      if (ks % kLoadEvery == 1 && ks / kLoadEvery < Fill<F>::kLoads) fill.issue(ks / kLoadEvery);
    }
    mfma_v_drain(s);
    __builtin_amdgcn_sched_barrier(0);
    // ---- softmax weights (log2 domain); reg r is token 8 (r / 4) + 4 hi + r % 4
    if ((k + 1) * kTileTok > limit_min) {  // the last tokens: the row's limit (and the sequence end)
      const int lt = limit - k * kTileTok;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * hi + (r & 3) >= lt) s[r] = -INFINITY;
    }
    if (k == k0 && !fixed) {  // a pass's reference: the first tile's max (uniform branch)
      float smax = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) smax = fmaxf(smax, s[r]);
      acc.m_ref = finite_ref(fmaxf(smax, wave_partner(smax)) * a.scale_log2 + kRefLift);
    }
    // the weights need only the fixed reference, not this tile's max.  Regs
    // r < 8 are the tokens of P.V k-step 0 (tokens 0..15): those weights come
    // first; the rest (and the max tracking) are computed between the MFMAs
    // of k-step 0.
    const float neg_ref = -acc.m_ref;
    float ps = 0.0f;
    unsigned phi[8], plo[8];  // packed bf16 pairs: P high part and remainder
    auto weights = [&](int r) {
      // v_exp_f32 directly: weights below 2^-126 of the reference flush to 0
      const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, neg_ref));
      const float pb = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], a.scale_log2, neg_ref));
      ps += pa + pb;
      const unsigned h2 = pack_bf16x2(pa, pb);
      phi[r >> 1] = h2;
      plo[r >> 1] = pack_bf16x2(pa - bf16_lo(h2), pb - bf16_hi(h2));
    };
#pragma unroll
    for (int r = 0; r < 8; r += 2) weights(r);
    // this tile's max (log2 units): tracks the split's true max and detects a
    // rise beyond 2^kMaxLift above the reference (the weights above may then
    // have overflowed: the pass is redone with the true max)
    auto track_max = [&]() {
      float smax = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) smax = fmaxf(smax, s[r]);
      const float mt = fmaxf(smax, wave_partner(smax)) * a.scale_log2;
      acc.m_seen = fmaxf(acc.m_seen, mt);
      lifted |= mt - acc.m_ref > kMaxLift;
    };
    // ---- O^T += khat^T . P  (k-step kk covers tile tokens 16 kk .. 16 kk + 15);
    //      the next tile's dequantization pieces are spread between the MFMAs
    const int nvalid_next = min(kTileTok, L - (k + 1) * kTileTok);
    constexpr int kSub = Fill<F>::kSubsteps;
    bf16x8 bp[2][2];  // [kk][hi/lo]
    bp[0][0] = __builtin_bit_cast(bf16x8, (u32x4){phi[0], phi[1], phi[2], phi[3]});
    bp[0][1] = __builtin_bit_cast(bf16x8, (u32x4){plo[0], plo[1], plo[2], plo[3]});
    // step = 16 kk + ct: A operand = khat^T for channels [32 ct, 32 ct + 32) and
    // the 16 tokens of k-step kk, read 3 steps ahead.  Scheduling fences pin
    // the order MFMA / VALU piece / MFMA / ..., so that the VALU work issues in
    // the shadow of the matrix pipe.
    const __bf16* vbase = tile + tr_row0 * kRow + 8 * tr_chunk + tr_half;
    auto tr_read = [&](int step) {
      const __bf16* v0 = vbase + 16 * (step >> 4) * kRow + 32 * (step & 15);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)v0);
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v0 + 2 * kRow));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 va[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) va[d] = tr_read(d);
#pragma unroll
    for (int step = 0; step < 32; ++step) {
      const int kk = step >> 4, ct = step & 15;
      if (step == 16) {
        bp[1][0] = __builtin_bit_cast(bf16x8, (u32x4){phi[4], phi[5], phi[6], phi[7]});
        bp[1][1] = __builtin_bit_cast(bf16x8, (u32x4){plo[4], plo[5], plo[6], plo[7]});
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        __builtin_amdgcn_sched_barrier(0);
        acc.o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[step % 3], bp[kk][h], acc.o[ct], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        const int slot = 2 * step + h;
        if (slot < 4) weights(8 + 2 * slot);       // weights of k-step 1
        if (slot == 5) track_max();
        const int u = slot - (64 - kSub);   // dequantization steps in the last kSub slots
        if (u >= 0 && u < kSub) fill.substep(next, nvalid_next, u);
      }
      if (step + 3 < 32) va[step % 3] = tr_read(step + 3);
    }
    acc.l_sum += ps;
    __builtin_amdgcn_sched_barrier(0);
    if (kSub == 0) fill.store(next, nvalid_next);
    __syncthreads();
  }
  return lifted;
}

// The same tile sequence for a wavefront that owns no rows (fewer than 32 w
// rows in the workgroup): it only helps fill the tiles and keeps the barrier
// sequence.
template <int F>
__device__ __forceinline__ void split_pass_fill_only(const DecodeArgs& a, __bf16* smem, const int32_t* bt, int L,
                                                     int k0, int k1) {
  PageWindow win(bt, k0, k1);
  Fill<F> fill;
  fill.load(a.cache, win.page_of(k0), k0 & 1, a.num_pages);
  fill.store(smem, min(kTileTok, L - k0 * kTileTok));
  __syncthreads();
  for (int k = k0; k < k1; ++k) {
    __bf16* next = smem + ((k - k0 + 1) & 1) * kTile;
    if (k + 1 < k1) {
      fill.load(a.cache, win.page_of(k + 1), (k + 1) & 1, a.num_pages);
      fill.store(next, min(kTileTok, L - (k + 1) * kTileTok));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- channel-split variant
// For <= 64 rows per sequence one head group per wavefront would leave two or
// three wavefronts (SIMDs) without MFMA work, and one tile in flight per
// compute unit keeps HBM far from busy.  Here the 4 wavefronts form 4 / C head
// groups of C wavefronts (the launcher uses C = 4 for <= 32 rows, C = 2 for
// 33..64); part c of a group takes
// k-steps [c NK, (c + 1) NK) of Q.K^T (NK = 36 / C, q entirely in registers)
// and channels [c 512 / C, (c + 1) 512 / C) of P.V (O in 256 / C
// accumulators).  The partial logits go through LDS as a reduce-scatter:
// wavefront c adds the C parts (in part order) for its 4 / C quarters of the
// tile only, computes their weights and publishes them as the P.V operand in
// LDS, which every wavefront of the group then reads; the denominators and
// maxima of the quarters are combined at the end of the pass, so all
// wavefronts of a group hold bitwise the same weights and denominator.  The
// packed bytes of the next D tiles are kept in registers (the launcher uses
// D = 1: at C = 4 the other workgroup on the compute unit covers the load
// latency).
template <int C> struct CsAcc {
  f32x16 o[16 / C];
  float l_sum, m_ref, m_seen;
};

constexpr int kXchFloats = 64 * 16;  // one wavefront's partial S^T block

template <int F, int C, int D>
__device__ __forceinline__ bool split_pass_cs(const DecodeArgs& a, __bf16* smem, const int32_t* bt, int L, int k0,
                                              int k1, const bf16x8 (&qr)[36 / C], int limit, bool fixed,
                                              float m_fixed, CsAcc<C>& acc) {
  const int limit_min = L - (a.s_q - 1);
  constexpr int NK = 36 / C, NCT = 16 / C;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hi = lane >> 5;
  const int part = wave % C, group = wave / C;
  // the partial logits go through the tile buffer that receives the next
  // tile: it is free from the end of the previous P.V until this tile's
  // dequantization starts (after the barrier that follows the weights), so
  // the pass needs only the two tile buffers and the weights blocks, and at
  // C = 4 two workgroups fit on a compute unit
  const int g = lane >> 4, i16 = lane & 15;
  const int tr_row0 = 4 * (i16 >> 2) + (g >> 1);
  const int tr_chunk = 2 * (g & 1) + ((i16 & 3) >> 1);
  const int tr_half = 4 * (i16 & 1);

#pragma unroll
  for (int i = 0; i < NCT; ++i) acc.o[i] = (f32x16){};
  acc.l_sum = 0.0f;
  acc.m_ref = fixed ? finite_ref(m_fixed) : -INFINITY;
  acc.m_seen = -INFINITY;
  bool lifted = false;

  PageWindow win(bt, k0, k1);
  {
    Fill<F> first;
    first.load(a.cache, win.page_of(k0), k0 & 1, a.num_pages);
    first.store(smem, min(kTileTok, L - k0 * kTileTok));
  }
  // ring: fr[j] holds the packed bytes of tile k + 1 while tile k (k - k0 = j
  // mod D) computes; tiles past the range reload the last one (harmless)
  Fill<F> fr[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int kt = min(k0 + 1 + j, k1 - 1);
    fr[j].load(a.cache, win.page_of(kt), kt & 1, a.num_pages);
  }
  __syncthreads();

  for (int kb = k0; kb < k1; kb += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int k = kb + j;
      if (k >= k1) break;  // uniform
      __bf16* tile = smem + ((k - k0) & 1) * kTile;
      __bf16* next = smem + ((k - k0 + 1) & 1) * kTile;
      // ---- partial S^T over this part's k-steps, operands read 4 ahead
      f32x16 s = {};
      const __bf16* arow = tile + rho(lane & 31) * kRow + 8 * hi + 16 * (part * NK);
      bf16x8 kv[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) kv[d] = *(const bf16x8*)(arow + 16 * d);
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[i & 3], qr[i], s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 4 < NK) kv[i & 3] = *(const bf16x8*)(arow + 16 * (i + 4));
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- reduce-scatter of the partial logits: wavefront `part` adds the C
      //      parts (in part order) for the quarters j4 = QPW part .. QPW part +
      //      QPW - 1 only (accumulator regs 4 j4 .. 4 j4 + 3: tokens 8 j4 + 4 hi +
      //      [0, 4) of its lane's head) and computes their weights
      constexpr int QPW = 4 / C;  // quarters of the tile per wavefront
      float* xch = (float*)next;  // [wave][4][lane][4] floats
      {
        float* xw = xch + wave * kXchFloats + 4 * lane;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) *(f32x4*)(xw + 256 * j4) = (f32x4){s[4 * j4], s[4 * j4 + 1], s[4 * j4 + 2], s[4 * j4 + 3]};
      }
      __syncthreads();
      const float* xg = xch + group * C * kXchFloats + 4 * lane;
      f32x4 sq[QPW];
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        const int j4 = QPW * part + qi;
        sq[qi] = *(const f32x4*)(xg + 256 * j4);
#pragma unroll
        for (int p = 1; p < C; ++p) sq[qi] += *(const f32x4*)(xg + p * kXchFloats + 256 * j4);
      }
      if (k == k0 && !fixed) {  // a pass's reference: the first tile's max over all its tokens
        float smax = -INFINITY;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          f32x4 v = *(const f32x4*)(xg + 256 * j4);
#pragma unroll
          for (int p = 1; p < C; ++p) v += *(const f32x4*)(xg + p * kXchFloats + 256 * j4);
          if ((k + 1) * kTileTok > limit_min) {
            const int lt = limit - k * kTileTok, lt_l = lt - 4 * hi;  // see the masking of the quarters below
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (C == 4 ? 8 * j4 + i >= lt_l : 8 * j4 + 4 * hi + i >= lt) v[i] = -INFINITY;
          }
          smax = fmaxf(smax, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
        }
        acc.m_ref = finite_ref(fmaxf(smax, wave_partner(smax)) * a.scale_log2 + kRefLift);
      }
      if ((k + 1) * kTileTok > limit_min) {  // the last tokens: the row's limit (and the sequence end)
        const int lt = limit - k * kTileTok;
        // at C = 4 (256 registers per wavefront) per-lane token indices would
        // be hoisted out of the loop and spilled: compare one per-lane bound
        // against compile-time offsets there
        const int lt_l = lt - 4 * hi - 8 * QPW * part;
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (C == 4 ? 8 * qi + i >= lt_l : 8 * (QPW * part + qi) + 4 * hi + i >= lt) sq[qi][i] = -INFINITY;
      }
      const float neg_ref = -acc.m_ref;
      // publish the weights as the P.V operand: bp[kk][h] of a lane holds regs
      // 8 kk .. 8 kk + 7 of that lane, so quarter j4 is its slots
      // 4 (j4 & 1) .. + 3 of k-step j4 / 2 (hi and lo halves)
      unsigned char* pbuf = (unsigned char*)(smem + 2 * kTile) + 4096 * group;  // per group: [kk][h][lane][8 bf16]
      float smax = -INFINITY;
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        float pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[qi][i], a.scale_log2, neg_ref));
        acc.l_sum += (pw[0] + pw[1]) + (pw[2] + pw[3]);
        smax = fmaxf(smax, fmaxf(fmaxf(sq[qi][0], sq[qi][1]), fmaxf(sq[qi][2], sq[qi][3])));
        const unsigned h01 = pack_bf16x2(pw[0], pw[1]), h23 = pack_bf16x2(pw[2], pw[3]);
        const unsigned l01 = pack_bf16x2(pw[0] - bf16_lo(h01), pw[1] - bf16_hi(h01));
        const unsigned l23 = pack_bf16x2(pw[2] - bf16_lo(h23), pw[3] - bf16_hi(h23));
        const int j4 = QPW * part + qi, kk = j4 >> 1, off = 8 * (j4 & 1) + 16 * lane;
        *(u32x2*)(pbuf + (2 * kk) * 1024 + off) = (u32x2){h01, h23};
        *(u32x2*)(pbuf + (2 * kk + 1) * 1024 + off) = (u32x2){l01, l23};
      }
      {
        const float mt = fmaxf(smax, wave_partner(smax)) * a.scale_log2;
        acc.m_seen = fmaxf(acc.m_seen, mt);
        lifted |= mt - acc.m_ref > kMaxLift;
      }
      __syncthreads();  // weights published; every wavefront is past its exchange reads
      // ---- O^T (this part's channels) += khat^T . P, next tile's dequant between the MFMAs
      const int nvalid_next = min(kTileTok, L - (k + 1) * kTileTok);
      constexpr int kPvH = 2;  // P.V MFMAs per step: high and low weights
      constexpr int kSub = Fill<F>::kSubsteps;
      constexpr int kSlots = 2 * kPvH * NCT;                 // MFMAs of this phase
      constexpr int kPer = kSub ? (kSub + kSlots - 1) / kSlots : 1;  // dequant steps per MFMA slot
      constexpr int kFirst = kSlots - (kSub + kPer - 1) / kPer;     // first slot that carries steps
      bf16x8 bp[2][kPvH];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int h = 0; h < kPvH; ++h) bp[kk][h] = *(const bf16x8*)(pbuf + (2 * kk + h) * 1024 + 16 * lane);
      const __bf16* vbase = tile + tr_row0 * kRow + 8 * tr_chunk + tr_half + 32 * (part * NCT);
      auto tr_read = [&](int step) {  // step = NCT kk + ct (ct relative to this part)
        const __bf16* v0 = vbase + 16 * (step / NCT) * kRow + 32 * (step % NCT);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)v0);
        const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v0 + 2 * kRow));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 va[3];
#pragma unroll
      for (int d = 0; d < 3; ++d) va[d] = tr_read(d);
#pragma unroll
      for (int step = 0; step < 2 * NCT; ++step) {
        const int kk = step / NCT, ct = step % NCT;
#pragma unroll
        for (int h = 0; h < kPvH; ++h) {
          __builtin_amdgcn_sched_barrier(0);
          acc.o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[step % 3], bp[kk][h], acc.o[ct], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          const int slot = kPvH * step + h - kFirst;
#pragma unroll
          for (int e = 0; e < kPer; ++e) {
            const int u = slot * kPer + e;
            if (slot >= 0 && u < kSub) fr[j].substep(next, nvalid_next, u);
          }
        }
        if (step + 3 < 2 * NCT) va[step % 3] = tr_read(step + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kSub == 0) fr[j].store(next, nvalid_next);
      // the ring slot is free again: packed bytes of tile k + 1 + D
      {
        const int kt = min(k + 1 + D, k1 - 1);
        fr[j].load(a.cache, win.page_of(kt), kt & 1, a.num_pages);
      }
      __syncthreads();
    }
  }
  // each wavefront summed and tracked only its quarter of every tile: combine
  // the group's denominators (in part order, the same in every wavefront) and
  // maxima through LDS (the tile buffers are free after the last barrier)
  {
    float* ex = (float*)smem;  // [wave][lane] sums, then [wave][lane] maxima
    ex[wave * 64 + lane] = acc.l_sum;
    ex[256 + wave * 64 + lane] = acc.m_seen;
    __syncthreads();
    float l = ex[group * C * 64 + lane], m = ex[256 + group * C * 64 + lane];
#pragma unroll
    for (int p = 1; p < C; ++p) {
      l += ex[(group * C + p) * 64 + lane];
      m = fmaxf(m, ex[256 + (group * C + p) * 64 + lane]);
    }
    acc.l_sum = l;
    acc.m_seen = m;
  }
  return lifted;
}

template <bool kDirect, int C>
__device__ __forceinline__ void write_split_cs(const DecodeArgs& a, int b, int64_t slot, const RowOf& row,
                                               CsAcc<C>& acc) {
  constexpr int NCT = 16 / C;
  const int hi = (threadIdx.x & 63) >> 5, part = (threadIdx.x >> 6) % C;
  const float l_tot = acc.l_sum + wave_partner(acc.l_sum);
  // a row that sees no token of the piece: output 0, lse -inf
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse = l_tot > 0.0f ? (acc.m_ref + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  const int R = a.heads, head = row.g;
  if (!row.valid) return;
  if (kDirect) {
    __bf16* orow = a.out + ((int64_t)b * R + head) * kDc + 4 * hi + 32 * (part * NCT);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const unsigned w0 = pack_bf16x2(acc.o[ct][4 * rq] * inv, acc.o[ct][4 * rq + 1] * inv);
        const unsigned w1 = pack_bf16x2(acc.o[ct][4 * rq + 2] * inv, acc.o[ct][4 * rq + 3] * inv);
        *(uint2*)(orow + 32 * ct + 8 * rq) = make_uint2(w0, w1);
      }
    if (a.lse_out && hi == 0 && part == 0) a.lse_out[b * R + head] = lse;
  } else {
    const int64_t prow = slot * R + head;
    float* orow = a.o_part + prow * kDc + 4 * hi + 32 * (part * NCT);
    // the four stores of a channel tile fill its 128-byte lines of the 32
    // rows: kept together (the fences stop the scheduler from interleaving
    // the tiles), a line is complete before the write burst at the end of
    // the kernel can evict it half written, which doubled the bytes written
    // to HBM at 64 heads
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x4 v = {acc.o[ct][4 * rq] * inv, acc.o[ct][4 * rq + 1] * inv, acc.o[ct][4 * rq + 2] * inv,
                         acc.o[ct][4 * rq + 3] * inv};
        *(f32x4*)(orow + 32 * ct + 8 * rq) = v;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (hi == 0 && part == 0) a.lse_part[prow] = lse;
  }
}

// Writes one pass result: the final bf16 output (direct mode) or an fp32
// partial row at a.o_part[prow * 512] / a.lse_part[prow] (prow = slot * R + row).
template <bool kDirect>
__device__ __forceinline__ void write_split(const DecodeArgs& a, int b, int64_t slot, const RowOf& row,
                                            const SplitAcc& acc) {
  const int hi = (threadIdx.x & 63) >> 5;
  const float l_tot = acc.l_sum + wave_partner(acc.l_sum);
  // a row that sees no token of the piece: output 0, lse -inf
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse = l_tot > 0.0f ? (acc.m_ref + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  const int R = a.heads, head = row.g;
  if (!row.valid) return;
  if (kDirect) {
    __bf16* orow = a.out + ((int64_t)b * R + head) * kDc + 4 * hi;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const unsigned w0 = pack_bf16x2(acc.o[ct][4 * rq] * inv, acc.o[ct][4 * rq + 1] * inv);
        const unsigned w1 = pack_bf16x2(acc.o[ct][4 * rq + 2] * inv, acc.o[ct][4 * rq + 3] * inv);
        *(uint2*)(orow + 32 * ct + 8 * rq) = make_uint2(w0, w1);
      }
    if (a.lse_out && hi == 0) a.lse_out[b * R + head] = lse;
  } else {
    const int64_t prow = slot * R + head;
    float* orow = a.o_part + prow * kDc + 4 * hi;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x4 v = {acc.o[ct][4 * rq] * inv, acc.o[ct][4 * rq + 1] * inv, acc.o[ct][4 * rq + 2] * inv,
                         acc.o[ct][4 * rq + 3] * inv};
        *(f32x4*)(orow + 32 * ct + 8 * rq) = v;
      }
    if (hi == 0) a.lse_part[prow] = lse;
  }
}

// ---------------------------------------------------------------- independent wavefronts (<= 16 rows)
// At <= 16 rows per sequence one 16 x 16 MFMA block holds every row, so a
// wavefront can carry its own tokens through the whole attention step.  Four
// wavefronts per workgroup (one per SIMD, one workgroup per compute unit)
// take every fourth 32-token tile of the piece; a tile is two 16-token
// blocks b = 0, 1.  Each wavefront, per tile:
//   1. loads the tile's packed bytes while the previous tile computes; lane
//      (t, g) = (lane % 16, lane / 16) owns token t of both blocks and a
//      quarter of their channels: the 8 values of k-step ks that Q.K^T needs
//      in its lane (channels iw_chan(ks, g) .. + 8) are one code dword;
//   2. dequantizes k-step by k-step in registers, straight into the A operand
//      of MFMA 16x16x32 bf16 (16 tokens x 32 channels), one MFMA per block
//      sharing B = q^T (the rows of the piece are loaded from global memory
//      once per pass and held in registers); the content values also go
//      to the wavefront's own LDS buffer for step 4.  Output: S^T, lane (h, g) holding row h for tokens
//      4 g .. 4 g + 3 of each block;
//   3. takes the eight softmax weights of its lane against a fixed reference
//      per wavefront and pass (as in split_pass) and splits them into high
//      and low bf16 halves: the lane's weights are already its slots of the
//      P.V operand (k slots 0..3: block 0 tokens 4 g + [0, 4), slots 4..7: block
//      1 tokens 4 g + [0, 4));
//   4. P.V on MFMA 16x16x32 bf16 with k = the tile's 32 tokens: A = V^T (16
//      channels x 32 tokens) from two transposing LDS reads of its buffer,
//      one MFMA with the high and one with the low weights, O^T (512 channels
//      x 16 rows) in 32 x 4 accumulators.
// Software pipelining: the P.V of tile i runs between the Q.K^T k-steps of
// tile i + 1.  No barrier is taken per tile.  At the end of a piece the four
// partial results (each against its own reference) are merged through LDS
// with log-sum-exp weights.
constexpr int kIwWaves = 4;
constexpr int kIwThreads = 64 * kIwWaves;
constexpr int kIwTok = 32;                        // tokens per tile of a wavefront
constexpr int kVRow = kDc + 16;                   // bf16 per row of a V buffer (1056 bytes; see vrow)
constexpr int kVBuf = kIwTok * kVRow;             // bf16 per wavefront buffer
constexpr int kIwRedRow = kDc + 4;                // fp32 per row in the end-of-piece merge
constexpr size_t kIwRedOff = (size_t)kIwWaves * kVBuf * sizeof(__bf16);  // 135168 bytes
static_assert(kIwWaves * 16 * kIwRedRow * sizeof(float) <= (size_t)kIwWaves * kVBuf * sizeof(__bf16),
              "the wavefronts' outputs fit in the V buffers");

// value of lane l ^ 16 / l ^ 32 (through ds_bpermute; used a few times per pass)
__device__ __forceinline__ float lane_xor(float v, int m) {
  return __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, v), m));
}

// 8 INT4 codes of a dword (element e in bits 4 e) -> bf16(fma(code, S, Z));
// s24 = 2^24 S, s20 = 2^20 S, Z the high half of `sz`.  Elements 0, 4 sit at
// bits 0, 16 (against s24), 1, 5 at bits 4, 20 (s20); 2, 6 and 3, 7 likewise
// after a shift by 8.
__device__ __forceinline__ bf16x8 dq_int4x8(unsigned w, float s24, float s20, unsigned sz) {
  const h2 a = as_h2(mask_bytes(w, 0x000F000Fu)), b = as_h2(mask_bytes(w, 0x00F000F0u));
  const unsigned w8 = w >> 8;
  const h2 c = as_h2(mask_bytes(w8, 0x000F000Fu)), d = as_h2(mask_bytes(w8, 0x00F000F0u));
  const u32x4 o = {pack_bf16x2(dq_sub(a[0], s24, sz), dq_sub(b[0], s20, sz)),
                   pack_bf16x2(dq_sub(c[0], s24, sz), dq_sub(d[0], s20, sz)),
                   pack_bf16x2(dq_sub(a[1], s24, sz), dq_sub(b[1], s20, sz)),
                   pack_bf16x2(dq_sub(c[1], s24, sz), dq_sub(d[1], s20, sz))};
  return __builtin_bit_cast(bf16x8, o);
}
__device__ __forceinline__ bf16x8 dq_int2x8(const unsigned (&m)[8], int hf, const SzScaled<4>& z) {
  float e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = dq_sub(as_h2(m[j])[hf], z.s[j % 4], z.sz);
  const u32x4 o = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
  return __builtin_bit_cast(bf16x8, o);
}

// Packed bytes of one lane's share of a 16-token block (token t of the block,
// lane group g) and the dequantization of its k-steps.  Both formats give
// lane group g the same channels: content k-step ks = 4 m + d (block m of 128
// channels) holds channels 128 m + 32 g + 8 d .. + 8 of the lane's token, and
// RoPE k-steps 16, 17 hold channels 512 + 32 (ks - 16) + 8 g .. + 8
// (iw_chan).  The q operand and the V buffer use the same offsets.  The
// registers hold one block: part i (content block m = i, or the RoPE part
// i = 4) is reloaded with the next tile's bytes right after its last k-step,
// so the loads of the next tile are in flight while this one computes.
// Addresses: a wavefront-uniform page base plus per-lane offsets fixed for
// the pass; `hp` is the block's quarter of its page.
__device__ __forceinline__ constexpr int iw_chan(int ks, int g) {
  return ks < 16 ? 128 * (ks >> 2) + 32 * g + 8 * (ks & 3) : kDc + 32 * (ks - 16) + 8 * g;
}

// Per-lane byte offsets within a page: content codes, content S/Z, RoPE codes,
// RoPE S/Z.  The loads are buffer loads: the page is a buffer resource in
// scalar registers (built once per tile), the uniform part of each offset a
// scalar or immediate, and only this 32-bit offset lives per lane, so no load
// needs 64-bit address arithmetic in the vector ALU (and none can leave the
// page: bytes past the resource's size read as zero).
struct SubLanes {
  unsigned c, sz, rc, rsz;
};
// word 3 of a gfx9 buffer resource: 32-bit data format, no swizzle, no stride
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* page_base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(page_base), 0, bytes, kBufWord3);
}

template <int F> struct SubFill;

template <> struct SubFill<kC4R4> {
  using Lay = PageLayout<kC4R4>;
  // block m of lane group g: chunk 4 m + g (16 bytes: 32 channels), group 2 m + g / 2
  static __device__ __forceinline__ SubLanes lanes(unsigned t, unsigned g) {
    return SubLanes{16 * t + 1024 * g, 4 * t + 256 * (g >> 1), 16 * t + 4 * g, 4 * t};
  }
  u32x4 c[4];
  unsigned sz[4];
  unsigned r[2];    // dword g of RoPE chunks 0, 1
  unsigned rsz;
  __device__ __forceinline__ void issue(int i, __amdgpu_buffer_rsrc_t pg, int hp, const SubLanes& o) {
    if (i < 4) {
      c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pg, o.c, Lay::kCodesA + 256 * hp + 4096 * i, 0));
      sz[i] = __builtin_amdgcn_raw_buffer_load_b32(pg, o.sz, Lay::kSzB + 64 * hp + 512 * i, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        r[j] = __builtin_amdgcn_raw_buffer_load_b32(pg, o.rc, Lay::kCodesC + 256 * hp + 1024 * j, 0);
      rsz = __builtin_amdgcn_raw_buffer_load_b32(pg, o.rsz, Lay::kSzD + 64 * hp, 0);
    }
  }
  using Sz = SzScaled<2>;
  __device__ __forceinline__ Sz sz_of(int ks, bool live) const {
    return sz_scaled<2, 4>(live ? (ks < 16 ? sz[ks >> 2] : rsz) : 0u);
  }
  __device__ __forceinline__ bf16x8 step(int ks, const Sz& z) {
    return dq_int4x8(ks < 16 ? c[ks >> 2][ks & 3] : r[ks - 16], z.s[0], z.s[1], z.sz);
  }
};

template <> struct SubFill<kC2R4> {
  using Lay = PageLayout<kC2R4>;
  // block m of lane group g: bytes 8 (g & 1) .. + 8 of chunk 2 m + g / 2 (32
  // channels), group 4 m + g
  static __device__ __forceinline__ SubLanes lanes(unsigned t, unsigned g) {
    return SubLanes{16 * t + 1024 * (g >> 1) + 8 * (g & 1), 4 * t + 256 * g, 16 * t + 4 * g, 4 * t};
  }
  u32x2 c[4];
  unsigned sz[4];
  unsigned r[2];
  unsigned rsz;
  unsigned m[8];    // the dword being converted, split as int2_split does
  __device__ __forceinline__ void issue(int i, __amdgpu_buffer_rsrc_t pg, int hp, const SubLanes& o) {
    if (i < 4) {
      c[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(pg, o.c, Lay::kCodesA + 256 * hp + 2048 * i, 0));
      sz[i] = __builtin_amdgcn_raw_buffer_load_b32(pg, o.sz, Lay::kSzB + 64 * hp + 1024 * i, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        r[j] = __builtin_amdgcn_raw_buffer_load_b32(pg, o.rc, Lay::kCodesC + 256 * hp + 1024 * j, 0);
      rsz = __builtin_amdgcn_raw_buffer_load_b32(pg, o.rsz, Lay::kSzD + 64 * hp, 0);
    }
  }
  using Sz = SzScaled<4>;   // 2^24 S, 2^22 S, 2^20 S, 2^18 S (the RoPE codes use 2^24 S and 2^20 S)
  __device__ __forceinline__ Sz sz_of(int ks, bool live) const {
    return sz_scaled<4, 2>(live ? (ks < 16 ? sz[ks >> 2] : rsz) : 0u);
  }
  // k-step 4 m + d: half d & 1 of dword d / 2 of block m
  __device__ __forceinline__ bf16x8 step(int ks, const Sz& z) {
    if (ks >= 16) return dq_int4x8(r[ks - 16], z.s[0], z.s[2], z.sz);
    if ((ks & 1) == 0) int2_split(c[ks >> 2][(ks & 3) >> 1], m);
    return dq_int2x8(m, ks & 1, z);
  }
};

struct IwAcc {
  f32x4 o[32];   // o[ct][r]: O^T[16 ct + 4 g + r][lane's row], against 2^m_ref
  float l_sum;   // this lane's tokens' share of sum_t p_t
  float m_ref;   // reference (log2 units) of this wavefront's weights
  float m_seen;  // max logit (log2 units) of this lane's tokens
};

// Row r of a wavefront's V buffer (token r of the tile) starts at element
// vrow(r): rows 528 bf16 (1056 bytes) apart, rows 8..15 and 24..31 shifted by
// 16 bytes.  In rows whose bit 2 is set (vswap) the two 16-byte halves of
// every 32-byte channel pair trade places.  The LDS serves 16-byte writes
// eight lanes at a time over 32 four-byte banks and reads 256 bytes at a time
// over 64 banks (the bank-conflict counter of this kernel and of the >16-row
// kernels shows both); with this layout the 8 rows of an 8-lane write group
// and the 8 rows x 32 bytes of a 32-lane transposing read each cover
// distinct banks, which no layout with one shift per row achieves.
__device__ __forceinline__ constexpr int vrow(int r) { return r * kVRow + 8 * ((r >> 3) & 1); }
__device__ __forceinline__ constexpr int vswap(int r) { return (r >> 2) & 1; }

// Q.K^T k-step order: the RoPE k-steps first (they write no V), then the
// content blocks in channel order.
__device__ __forceinline__ constexpr int iw_ks(int p) { return p < 2 ? 16 + p : p - 2; }
// P.V channel tiles issued with Q.K^T step p of the next tile: 4 each with
// the RoPE steps (channel block 0), then 2 per content step of channel
// blocks 0..2 (the tiles of block m + 1), none during block 3.  Every tile of
// channel block m is read before step 2 + 4 m writes block m of the next tile.
__device__ __forceinline__ constexpr int pv_begin(int p) { return p < 2 ? 4 * p : p < 14 ? 8 + 2 * (p - 2) : 32; }
__device__ __forceinline__ constexpr int pv_end(int p) { return p < 2 ? 4 * p + 4 : p < 14 ? 10 + 2 * (p - 2) : 32; }

// One pass of wavefront `wave` over its tiles u0 + wave + 4 i < u1 of the
// piece (32-token tiles), software-pipelined: the P.V of tile i runs between
// the Q.K^T k-steps of tile i + 1.  Returns true if a weight may have
// overflowed (a logit more than kMaxLift above the reference): the caller
// redoes the piece with a fixed reference.
template <int F>
__device__ __forceinline__ bool iw_pass(const DecodeArgs& a, __bf16* smem, const int32_t* bt, const __bf16* qg, int L,
                                        int u0, int u1, int limit, bool fixed, float m_fixed, IwAcc& acc) {
  using SF = SubFill<F>;
  const int limit_min = L - (a.s_q - 1);
  // the wavefront index as a scalar: tile indices, page offsets and load
  // offsets derived from it stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t = lane & 15, g = lane >> 4;  // QK operand lane: token t, channel quarter g; S^T lane: row t, tokens 4 g..
  __bf16* __restrict__ vbuf = smem + wave * kVBuf;
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) acc.o[ct] = (f32x4){};
  acc.l_sum = 0.0f;
  acc.m_ref = fixed ? finite_ref(m_fixed) : -INFINITY;
  acc.m_seen = -INFINITY;
  bool lifted = false;
  bool first = !fixed;
  const int ufirst = u0 + wave;
  if (ufirst >= u1) return false;
  PageWindow win(bt, ufirst, u1);
  // transposing-read addresses of the P.V operand: lane block kg = lane / 16
  // reads tokens 4 kg + j of block 0 (then of block 1), lane 4 j + r of the
  // block channels 4 r .. + 4 of the channel tile; lane i of the block
  // receives channel i of those 4 tokens
  const int trow = 4 * g + ((lane & 15) >> 2);
  const __bf16* __restrict__ vtr = vbuf + vrow(trow) + 8 * (((lane & 3) >> 1) ^ vswap(trow)) + 4 * (lane & 1);
  auto tr_read = [&](int ct) {
    const __bf16* v0 = vtr + 16 * ct;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)v0);
    const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v0 + vrow(16)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // the lane's rows t and 16 + t; even / odd 16-byte chunks of its channels
  // land one chunk up / down in swapped rows
  __bf16* __restrict__ vw0e = vbuf + vrow(t) + 8 * vswap(t);
  __bf16* __restrict__ vw0o = vbuf + vrow(t) - 8 * vswap(t);
  constexpr int kVw1 = vrow(16) - vrow(0);   // vrow(16 + t) - vrow(t), vswap alike
  const SubLanes lo = SF::lanes(t, g);

  SF f0, f1;  // blocks 0 and 1 of the tile
  __amdgpu_buffer_rsrc_t pg = page_rsrc(a.cache, PageLayout<F>::kBytes);
  int hpt = 0;   // half of the page of the tile whose bytes issue() loads next
  int pg_next = win.page_of(ufirst);
  auto aim = [&](int page, int u) {
    page = __builtin_amdgcn_readfirstlane(page);  // uniform: keeps the resource in scalar registers
    const bool ok = page >= 0 && page < a.num_pages;
    // an invalid page id gets an empty resource: its loads read zeros (codes
    // 0, S = Z = 0), so its rows dequantize to exact zeros
    pg = page_rsrc(a.cache + (ok ? page : 0) * (int64_t)PageLayout<F>::kBytes, ok ? PageLayout<F>::kBytes : 0);
    hpt = u & 1;
  };
  auto issue = [&](int i) {
    f0.issue(i, pg, 2 * hpt, lo);
    f1.issue(i, pg, 2 * hpt + 1, lo);
  };
  aim(pg_next, ufirst);
#pragma unroll
  for (int i = 0; i < 5; ++i) issue(i);

  // ---- Q.K^T state of the tile being dequantized
  f32x4 s0, s1;
  // the q operand of every k-step stays in registers for the pass (72 of
  // them: one wavefront per SIMD leaves room), loaded once from global
  // memory behind the first tile's loads, so both latencies overlap (qg: the
  // lane's q row, null for a row without a head: zeros)
  bf16x8 qall[18];
#pragma unroll
  for (int d = 0; d < 18; ++d) qall[d] = qg ? *(const bf16x8*)(qg + iw_chan(iw_ks(d), g)) : (bf16x8){};
  typename SF::Sz SZ0, SZ1;  // (S, Z) of the current group of each block
  bool live0 = false, live1 = false;
  auto qk_begin = [&](int u) {
    const bool ok = pg_next >= 0 && pg_next < a.num_pages;
    live0 = ok && kIwTok * u + t < L;
    live1 = ok && kIwTok * u + 16 + t < L;
    const int un = u + kIwWaves < u1 ? u + kIwWaves : u;  // the last one reloads itself: harmless
    pg_next = win.page_of(un);
    aim(pg_next, un);
    s0 = (f32x4){};
    s1 = (f32x4){};
  };
  // rows past the sequence end are zeroed through S = Z = 0; only tiles that
  // may hold such rows (kMask) pay for the selects
  auto qk_step = [&](int p, auto kMask) {
    constexpr bool kM = decltype(kMask)::value;
    const int ks = iw_ks(p);
    if (ks % 4 == 0 || ks == 16) {
      SZ0 = f0.sz_of(ks, !kM || live0);
      SZ1 = f1.sz_of(ks, !kM || live1);
    }
    const bf16x8 k0 = f0.step(ks, SZ0);
    const bf16x8 k1 = f1.step(ks, SZ1);
    const bf16x8 qk = qall[p];
    if (ks < 16) {
      __bf16* vw = (ks & 1) ? vw0o : vw0e;  // chunk iw_chan / 8 has the parity of ks
      *(bf16x8*)(vw + iw_chan(ks, g)) = k0;
      *(bf16x8*)(vw + kVw1 + iw_chan(ks, g)) = k1;
    }
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qk, s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qk, s1, 0, 0, 0);
    if (p == 1) issue(4);                              // RoPE part consumed
    if (p >= 2 && (ks & 3) == 3) issue(ks >> 2);       // content block consumed
  };
  // ---- softmax of a finished Q.K^T: weights against the reference, high /
  //      low bf16 halves, already in the lane's slots of the P.V operand
  bf16x8 bph, bpl;
  // kMask: the tile may hold tokens past a row's limit (or the sequence
  // end); the loop below runs the tiles that cannot with kMask = false, so
  // the compares and selects are not executed on every tile
  auto softmax = [&](int u, auto kMask) {
    f32x4 s[2] = {s0, s1};
    if (decltype(kMask)::value && kIwTok * (u + 1) > limit_min) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int lt = limit - kIwTok * u - 16 * b - 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r >= lt) s[b][r] = -INFINITY;
      }
    }
    const float smax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                             fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    if (first) {  // this wavefront's reference: its first tile's max (over the 32 tokens), lifted
      float m = fmaxf(smax, lane_xor(smax, 16));
      m = fmaxf(m, lane_xor(m, 32));
      acc.m_ref = finite_ref(m * a.scale_log2 + kRefLift);
      first = false;
    }
    {
      const float mt = smax * a.scale_log2;
      acc.m_seen = fmaxf(acc.m_seen, mt);
      lifted |= mt - acc.m_ref > kMaxLift;
    }
    const float neg_ref = -acc.m_ref;
    unsigned hw[4], lw[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], a.scale_log2, neg_ref));
      acc.l_sum += (p[0] + p[1]) + (p[2] + p[3]);
      hw[2 * b] = pack_bf16x2(p[0], p[1]);
      hw[2 * b + 1] = pack_bf16x2(p[2], p[3]);
      lw[2 * b] = pack_bf16x2(p[0] - bf16_lo(hw[2 * b]), p[1] - bf16_hi(hw[2 * b]));
      lw[2 * b + 1] = pack_bf16x2(p[2] - bf16_lo(hw[2 * b + 1]), p[3] - bf16_hi(hw[2 * b + 1]));
    }
    bph = __builtin_bit_cast(bf16x8, (u32x4){hw[0], hw[1], hw[2], hw[3]});
    bpl = __builtin_bit_cast(bf16x8, (u32x4){lw[0], lw[1], lw[2], lw[3]});
  };
  // ---- P.V of the previous tile: O^T += V^T . P_hi + V^T . P_lo, channel
  //      tile ct; operands read 3 tiles ahead, the low-weight MFMA of a tile
  //      issued after the high one of the next (no back-to-back accumulator)
  bf16x8 va[5];
  auto pv_start = [&]() {
#pragma unroll
    for (int d = 0; d < 3; ++d) va[d] = tr_read(d);
  };
  auto pv_tile = [&](int ct) {
    if (ct + 3 < 32) va[(ct + 3) % 5] = tr_read(ct + 3);
    acc.o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ct % 5], bph, acc.o[ct], 0, 0, 0);
    if (ct > 0) acc.o[ct - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[(ct - 1) % 5], bpl, acc.o[ct - 1], 0, 0, 0);
    if (ct == 31) acc.o[31] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[31 % 5], bpl, acc.o[31], 0, 0, 0);
  };

  // prologue: Q.K^T and weights of the first tile
  qk_begin(ufirst);
#pragma unroll
  for (int p = 0; p < 18; ++p) qk_step(p, std::true_type{});
  softmax(ufirst, std::true_type{});
  // P.V of tile u interleaved with Q.K^T of tile u + 4
  auto step_tile = [&](int u, auto kMask) {
    qk_begin(u + kIwWaves);
    pv_start();
#pragma unroll
    for (int p = 0; p < 18; ++p) {
      qk_step(p, kMask);
#pragma unroll
      for (int ct = pv_begin(p); ct < pv_end(p); ++ct) pv_tile(ct);
    }
    softmax(u + kIwWaves, kMask);
  };
  // tiles from u_mask on may hold tokens past a row's limit
  const int u_mask = limit_min >> 5;
  int u = ufirst;
  for (; u + kIwWaves < u1 && u + kIwWaves < u_mask; u += kIwWaves) step_tile(u, std::false_type{});
  for (; u + kIwWaves < u1; u += kIwWaves) step_tile(u, std::true_type{});
  // epilogue: P.V of the last tile
  pv_start();
#pragma unroll
  for (int ct = 0; ct < 32; ++ct) pv_tile(ct);
  return lifted;
}

// Merged result of a piece for the wavefronts' rows, written to `slot`
// (partials) or to the output (direct mode).  Per-wavefront reference,
// denominator and seen maximum come through `red`; the O blocks through the
// V buffers, each wavefront summing 128 of the 512 channels.
struct IwRed {
  float m[kIwWaves][16], l[kIwWaves][16], s[kIwWaves][16];
};
// V buffers, then the merge record
constexpr size_t kIwLds = kIwRedOff + sizeof(IwRed);

// Per-row totals of the piece: every lane of row t (lanes t, t + 16, t + 32,
// t + 48 of every wavefront) gets M = max reference, L = sum l 2^(m - M) and
// the seen maximum; also this wavefront's scale 2^(m_ref - M).
__device__ __forceinline__ void iw_totals(IwRed& red, const IwAcc& acc, float& M, float& Ltot, float& seen,
                                          float& f_own) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, t = lane & 15;
  float l = acc.l_sum + lane_xor(acc.l_sum, 16);
  l += lane_xor(l, 32);
  float sm = fmaxf(acc.m_seen, lane_xor(acc.m_seen, 16));
  sm = fmaxf(sm, lane_xor(sm, 32));
  if (lane < 16) {
    red.m[wave][t] = l > 0.0f ? acc.m_ref : -INFINITY;
    red.l[wave][t] = l;
    red.s[wave][t] = sm;
  }
  __syncthreads();
  M = -INFINITY;
  seen = -INFINITY;
#pragma unroll
  for (int w = 0; w < kIwWaves; ++w) {
    M = fmaxf(M, red.m[w][t]);
    seen = fmaxf(seen, red.s[w][t]);
  }
  Ltot = 0.0f;
  f_own = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kIwWaves; ++w)
      if (red.l[w][t] > 0.0f) Ltot += red.l[w][t] * __builtin_amdgcn_exp2f(red.m[w][t] - M);
    if (l > 0.0f) f_own = __builtin_amdgcn_exp2f(acc.m_ref - M);
  }
}

template <bool kDirect>
__device__ __forceinline__ void iw_write(const DecodeArgs& a, __bf16* smem, int b, int64_t slot, int chunk, int L,
                                         IwAcc& acc, float M, float f_own) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, t = lane & 15, g = lane >> 4;
  float* red = (float*)smem;  // kIwWaves x [16 rows][kIwRedRow] fp32 over the V buffers
  __syncthreads();            // the V buffers are free
  {
    float* dst = red + wave * 16 * kIwRedRow + t * kIwRedRow + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) *(f32x4*)(dst + 16 * ct) = acc.o[ct] * f_own;
  }
  __syncthreads();
  // this lane's summing share: row t, channels 128 wave + 32 g .. + 32
  f32x4 sum[8] = {};
#pragma unroll
  for (int src = 0; src < kIwWaves; ++src) {
    const float* s = red + src * 16 * kIwRedRow + t * kIwRedRow + 128 * wave + 32 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum[i] += *(const f32x4*)(s + 4 * i);
  }
  // row t of the workgroup: the totals are per row (any lane of row t holds them)
  const RowOf row = row_of(a, chunk, L, t);
  if (t >= a.s_q * a.chunk_heads || !row.valid) return;
  const float Ltot = acc.l_sum;  // (the caller stores the row total here)
  const float inv = Ltot > 0.0f ? 1.0f / Ltot : 0.0f;
  const float lse = Ltot > 0.0f ? (M + __log2f(Ltot)) * 0.69314718055994531f : -INFINITY;
  const int R = a.heads;
  const int ch = 128 * wave + 32 * g;
  if (kDirect) {
    __bf16* orow = a.out + ((int64_t)b * R + row.g) * kDc + ch;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x2 w = {pack_bf16x2(sum[2 * j][0] * inv, sum[2 * j][1] * inv),
                       pack_bf16x2(sum[2 * j][2] * inv, sum[2 * j][3] * inv)};
      const u32x2 x = {pack_bf16x2(sum[2 * j + 1][0] * inv, sum[2 * j + 1][1] * inv),
                       pack_bf16x2(sum[2 * j + 1][2] * inv, sum[2 * j + 1][3] * inv)};
      *(u32x4*)(orow + 8 * j) = (u32x4){w[0], w[1], x[0], x[1]};
    }
    if (a.lse_out && wave == 0 && g == 0) a.lse_out[b * R + row.g] = lse;
  } else {
    const int64_t prow = slot * R + row.g;
    float* orow = a.o_part + prow * kDc + ch;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(f32x4*)(orow + 4 * i) = sum[i] * inv;
    if (wave == 0 && g == 0) a.lse_part[prow] = lse;
  }
}

// Attention of sequence b over tiles [k0, k1) (32-token tiles, as
// process_range) with independent wavefronts; <= 16 rows.
template <int F, bool kDirect>
__device__ __forceinline__ void process_range_iw(const DecodeArgs& a, __bf16* smem, int b, int L, int k0, int k1,
                                                 int64_t slot, int chunk) {
  IwRed& red = *(IwRed*)((char*)smem + kIwRedOff);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = a.heads;
  const int rows = a.s_q * a.chunk_heads;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  // fused append: as process_range
  if (a.new_latent && k1 == (L + kTileTok - 1) / kTileTok && wave == 0) {
    const int64_t page = bt[(L - 1) / kPage];
    if (page >= 0 && page < a.num_pages)
      append_row<F>(a.new_latent + (int64_t)b * kDc, a.new_rope + (int64_t)b * kDr,
                    a.append_cache + page * (int64_t)PageLayout<F>::kBytes, (L - 1) % kPage);
    __threadfence();
  }
  __syncthreads();  // the previous piece (if any) has finished with LDS
  const RowOf row = row_of(a, chunk, L, lane & 15);
  const __bf16* qg = (lane & 15) < rows && row.valid ? a.q + ((int64_t)b * R + row.g) * kD : nullptr;
  const int limit = min(row.limit, L);
  const int u1 = min(k1, (L + kIwTok - 1) / kIwTok);
  bool fixed = false;
  float m_fixed = 0.0f;
  for (int pass = 0;; ++pass) {
    IwAcc acc;
    const bool lifted = iw_pass<F>(a, smem, bt, qg, L, k0, u1, limit, fixed, m_fixed, acc);
    const bool redo = __syncthreads_or(lifted);
    float M, Ltot, seen, f_own;
    iw_totals(red, acc, M, Ltot, seen, f_own);
    if (!redo || pass > 0) {
      acc.l_sum = Ltot;
      iw_write<kDirect>(a, smem, b, slot, chunk, L, acc, M, f_own);
      return;
    }
    fixed = true;
    m_fixed = seen;
    __syncthreads();  // every wavefront has read `red` before the next pass can rewrite it
  }
}

// Attention of sequence b over its tiles [k0, k1) (non-empty) for the rows of
// head chunk `chunk`, written to `slot`.  Called by every thread of the
// workgroup (uniform control flow).
template <int F, bool kDirect, int C>
__device__ __forceinline__ void process_range(const DecodeArgs& a, __bf16* smem, int b, int L, int k0, int k1,
                                              int64_t slot, int chunk) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = a.heads;                   // rows of the sequence
  const int rows = a.s_q * a.chunk_heads;  // rows of this workgroup
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  // fused append: the piece holding the sequence's last tile writes the new
  // token (position L - 1) first; the fence and the barrier below order the
  // write before any load of that page (no wavefront has read it yet)
  if (a.new_latent && k1 == (L + kTileTok - 1) / kTileTok && wave == 0) {
    const int64_t page = bt[(L - 1) / kPage];
    if (page >= 0 && page < a.num_pages)
      append_row<F>(a.new_latent + (int64_t)b * kDc, a.new_rope + (int64_t)b * kDr,
                    a.append_cache + page * (int64_t)PageLayout<F>::kBytes, (L - 1) % kPage);
    __threadfence();
  }
  __syncthreads();  // the previous range (if any) has finished with LDS
  if constexpr (C > 1) {
    // channel split: every wavefront has rows (the launcher picks C from the row count)
    constexpr int NK = 36 / C;
    const int part = wave % C, group = wave / C;
    const RowOf row = row_of(a, chunk, L, group * 32 + (lane & 31));
    const int hi = lane >> 5;
    bf16x8 qr[NK];
    {
      const __bf16* qh = a.q + ((int64_t)b * R + (row.valid ? row.g : 0)) * kD + 8 * hi + 16 * (part * NK);
      const bf16x8 zero = {};
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const bf16x8 v = *(const bf16x8*)(qh + 16 * i);
        qr[i] = row.valid ? v : zero;
      }
    }
    bool fixed = false;
    float m_fixed = 0.0f;
    for (int pass = 0;; ++pass) {
      CsAcc<C> acc;
      const bool lifted = split_pass_cs<F, C, 1>(a, smem, bt, L, k0, k1, qr, row.limit, fixed, m_fixed, acc);
      const bool redo = __syncthreads_or(lifted);
      if (!redo || pass > 0) {
        write_split_cs<kDirect, C>(a, b, slot, row, acc);
        return;
      }
      fixed = true;
      m_fixed = acc.m_seen;
    }
  } else {
    // stage the LDS k-steps of q (zeros for rows without a head): LDS chunk c
    // of row r holds channels 16 (2 (c / 2)) + 8 (c % 2) + [0, 8); the first
    // tile's barrier publishes it
    {
      __bf16* ql = smem + 2 * kTile;
      for (int ci = tid; ci < 128 * (kQLds / 8); ci += kThreads) {
        const int r = ci / (kQLds / 8), c = ci % (kQLds / 8);
        const RowOf qrow = row_of(a, chunk, L, r);
        bf16x8 v = {};
        if (r < rows && qrow.valid)
          v = *(const bf16x8*)(a.q + ((int64_t)b * R + qrow.g) * kD + 32 * (c >> 1) + 8 * (c & 1));
        *(bf16x8*)(ql + r * kQRow + 8 * c) = v;
      }
    }

    if (wave * 32 >= rows) {  // no rows for this wavefront: fill only (uniform per wave)
      for (int pass = 0;; ++pass) {
        split_pass_fill_only<F>(a, smem, bt, L, k0, k1);
        const bool redo = __syncthreads_or(0);
        if (!redo || pass > 0) return;
      }
    }

    const RowOf row = row_of(a, chunk, L, wave * 32 + (lane & 31));
    const int hi = lane >> 5;
    // q^T operand: lane holds row `row`, channels 16 ks + 8 hi + [0, 8) of the
    // register k-steps (odd ks < 32, and 32..35); the even ks < 32 are in LDS
    bf16x8 qr[kQRegSteps];
    {
      const __bf16* qh = a.q + ((int64_t)b * R + (row.valid ? row.g : 0)) * kD + 8 * hi;
      const bf16x8 zero = {};
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) {
        if (q_in_lds(ks)) continue;
        const bf16x8 v = *(const bf16x8*)(qh + 16 * ks);
        qr[q_reg_index(ks)] = row.valid ? v : zero;
      }
    }
    // pass 0 takes the first tile's max (plus kRefLift) as reference; a second
    // pass (only when a logit rises more than kRefLift + kMaxLift above that
    // max) uses the split's true max found by pass 0.
    bool fixed = false;
    float m_fixed = 0.0f;
    for (int pass = 0;; ++pass) {
      SplitAcc acc;
      const bool lifted = split_pass<F>(a, smem, bt, L, k0, k1, qr, row.limit, fixed, m_fixed, acc);
      const bool redo = __syncthreads_or(lifted);
      if (!redo || pass > 0) {
        write_split<kDirect>(a, b, slot, row, acc);
        return;
      }
      fixed = true;
      m_fixed = acc.m_seen;
    }
  }
}

__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int b) {
  const int L = a.seq_lens[b];
  return L < 0 ? 0 : (L > a.max_pages * kPage ? a.max_pages * kPage : L);
}

// Per-sequence splits: workgroup (split, b) covers pages [split * P, (split + 1) * P)
// of sequence b, the last split running to the end of the sequence.
// Threads of a decode workgroup: 256 (four wavefronts) in every variant.
template <int C> constexpr int decode_threads() { return C == 0 ? kIwThreads : kThreads; }

template <int F, bool kDirect, int C>
__device__ __forceinline__ void run_range(const DecodeArgs& a, __bf16* smem, int b, int L, int k0, int k1,
                                          int64_t slot, int chunk) {
  if constexpr (C == 0)
    process_range_iw<F, kDirect>(a, smem, b, L, k0, k1, slot, chunk);
  else
    process_range<F, kDirect, C>(a, smem, b, L, k0, k1, slot, chunk);
}

template <int F, bool kDirect, int C>
__global__ __launch_bounds__(decode_threads<C>(), C == 4 ? 2 : 1) void k_decode(const DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
  const int split = blockIdx.x, b = blockIdx.y, chunk = blockIdx.z;
  const int tid = threadIdx.x;
  const int R = a.heads;
  const int L = clamped_len(a, b);
  const int n_pages = (L + kPage - 1) / kPage;
  const int p0 = split * a.pages_per_split;
  const int p1 = (split == a.num_splits - 1) ? n_pages : min(p0 + a.pages_per_split, n_pages);
  if (p0 >= p1) {  // empty split: the chunk's rows get weight 0 (direct mode: output 0, lse -inf)
    const int rows = a.s_q * a.chunk_heads;
    for (int i = tid; i < rows * (kDirect ? kDc / 8 : 1); i += decode_threads<C>()) {
      const RowOf row = row_of(a, chunk, L, kDirect ? i / (kDc / 8) : i);
      if (!row.valid) continue;
      if (kDirect) {
        *(u32x4*)(a.out + ((int64_t)b * R + row.g) * kDc + 8 * (i % (kDc / 8))) = (u32x4){0u, 0u, 0u, 0u};
        if (a.lse_out && i % (kDc / 8) == 0) a.lse_out[b * R + row.g] = -INFINITY;
      } else {
        a.lse_part[((int64_t)b * a.num_splits + split) * R + row.g] = -INFINITY;
      }
    }
    return;
  }
  // tiles are half pages: tile k covers tokens [32 k, 32 k + 32)
  run_range<F, kDirect, C>(a, smem, b, L, 2 * p0, min(2 * p1, (L + kTileTok - 1) / kTileTok),
                           (int64_t)b * a.num_splits + split, chunk);
}

// Balanced partition: the batch's pages, laid end to end in sequence order
// (T pages), are cut into G = min(gridDim.x, T) equal shares, so that no
// share is empty; workgroup w < G takes pages [w T / G, (w + 1) T / G), which
// may span the end of one sequence and the start of others.  Each
// (workgroup, sequence) piece is written to partial slot w + b: the slots of
// one sequence are consecutive, and the workgroup holding a sequence's first
// page records (first slot, count) in a.meta[b].
// floor(w T / G) in double precision, exact here: w <= G <= 512 and T < 2^40
// pages (at most 65535 sequences of at most 2^24 pages) keep w T below 2^49,
// exact in a double, and a quotient that is not an integer lies at least 1 / G
// away from one, far beyond the division's rounding error (below 2^-13).
__device__ __forceinline__ int64_t share_start(int64_t w, int64_t T, int64_t G) {
  return (int64_t)floor((double)(w * T) / (double)G);
}

__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ unsigned long long uniform64(unsigned long long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Walk of the batch for one workgroup's share, kept in LDS: wavefront 0
// advances it between barriers, so no walk state stays in registers while
// the tiles run.  Sequences are taken 64 at a time (a "chunk"): their lengths,
// first-page offsets and which of them overlap the share.
struct FlatWalk {
  long long start, end;  // the share: pages [start, end)
  long long next;        // pages before the chunk after the current one
  unsigned long long mask;  // chunk sequences overlapping the share
  int b0, j;             // current chunk's first sequence; next index to look at
  int len[64];
  long long off[64];
  int piece[4];          // sequence (-1: share done), length, first tile, end tile
  int lens[kThreads];    // clamped lengths of sequences 0 .. kThreads - 1
};

// Clamped length of sequence b < a.batch: from the workgroup's copy for the
// first kThreads sequences, else from global memory.
__device__ __forceinline__ int walk_len(const DecodeArgs& a, const FlatWalk& walk, int b) {
  return b < kThreads ? walk.lens[b] : clamped_len(a, b);
}

// Wavefront 0 only (all 64 lanes): find the next piece of the share and
// publish it in walk.piece.  A sequence whose first page lies in the share
// gets its (first slot, slot count) recorded in meta.
__device__ __forceinline__ void flat_next_piece(const DecodeArgs& a, FlatWalk& walk, int64_t w, int64_t T,
                                                int64_t G) {
  const int ln = opaque_lane();
  const int64_t start = (int64_t)uniform64((unsigned long long)walk.start);
  const int64_t end = (int64_t)uniform64((unsigned long long)walk.end);
  int b0 = __builtin_amdgcn_readfirstlane(walk.b0), j = __builtin_amdgcn_readfirstlane(walk.j);
  unsigned long long mask = uniform64(walk.mask);
  int pb = -1, pl = 0, pk0 = 0, pk1 = 0;
  for (;;) {
    const unsigned long long m = j < 64 ? mask & (~0ull << j) : 0ull;
    if (m) {
      const int jj = __builtin_ctzll(m);
      const int L = __builtin_amdgcn_readfirstlane(walk.len[jj]);
      const int64_t off = (int64_t)uniform64((unsigned long long)walk.off[jj]);
      const int64_t n = (L + kPage - 1) / kPage;
      const int p0 = (int)((off > start ? off : start) - off);
      const int p1 = (int)((off + n < end ? off + n : end) - off);
      pb = b0 + jj;
      pl = L;
      pk0 = 2 * p0;
      pk1 = min(2 * p1, (L + kTileTok - 1) / kTileTok);
      j = jj + 1;
      break;
    }
    const int64_t base = (int64_t)uniform64((unsigned long long)walk.next);
    if (b0 + 64 >= a.batch || base >= end) break;  // the share is done
    b0 += 64;
    j = 0;
    // scan the chunk's page counts (inclusive prefix sum over the wavefront)
    const int b = b0 + ln;
    const int L = b < a.batch ? walk_len(a, walk, b) : 0;
    const int n = (L + kPage - 1) / kPage;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (ln >= d) incl += v;
    }
    const int64_t off = base + incl - n;
    const int64_t lo = off > start ? off : start;
    const int64_t hi = off + n < end ? off + n : end;
    const bool seg = b < a.batch && lo < hi;
    if (seg && off >= start && blockIdx.y == 0) {
      // the first page of b is in this share: b's slots run from w + b to
      // wl + b, wl the share holding b's last page
      const int64_t x = off + n - 1;
      int64_t wl = (x * G) / T;
      while (wl + 1 < G && share_start(wl + 1, T, G) <= x) ++wl;
      while (share_start(wl, T, G) > x) --wl;
      a.meta[2 * b] = (int)(w + b);
      a.meta[2 * b + 1] = (int)(wl - w + 1);
    }
    walk.len[ln] = L;
    walk.off[ln] = off;
    if (ln == 63) walk.next = base + incl;
    mask = __ballot(seg);
  }
  if (ln == 0) {
    walk.piece[0] = pb;
    walk.piece[1] = pl;
    walk.piece[2] = pk0;
    walk.piece[3] = pk1;
    walk.b0 = b0;
    walk.j = j;
    walk.mask = mask;
  }
}

template <int F, int C>
__global__ __launch_bounds__(decode_threads<C>(), C == 4 ? 2 : 1) void k_decode_flat(const DecodeArgs a) {
  constexpr int NT = decode_threads<C>();
  extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
  __shared__ unsigned long long s_total;
  __shared__ FlatWalk walk;
  const int tid = threadIdx.x;
  const int64_t w = blockIdx.x;
  // one read of the lengths: the first kThreads stay in LDS for the walk
  const int len_t = tid < a.batch ? clamped_len(a, tid) : 0;
  if (tid < kThreads) walk.lens[tid] = len_t;
  if (tid == 0) s_total = 0;
  __syncthreads();
  {
    unsigned long long part = (len_t + kPage - 1) / kPage;
    for (int b = tid + NT; b < a.batch; b += NT) part += (clamped_len(a, b) + kPage - 1) / kPage;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) part += __shfl_xor(part, d);
    if ((tid & 63) == 0) atomicAdd(&s_total, part);
  }
  __syncthreads();
  const int64_t T = (int64_t)uniform64(s_total);
  // empty sequences own no slots: record (0, 0) for them (strided over
  // workgroups; head chunk 0 writes all slot records)
  for (int b = (int)w * NT + tid; blockIdx.y == 0 && b < a.batch; b += (int)gridDim.x * NT)
    if ((b == tid ? len_t : clamped_len(a, b)) == 0) {
      a.meta[2 * b] = 0;
      a.meta[2 * b + 1] = 0;
    }
  const int64_t G = T < (int64_t)gridDim.x ? T : (int64_t)gridDim.x;
  if (w >= G) return;  // uniform: no share for this workgroup (or no pages at all)
  if (tid == 0) {
    walk.start = share_start(w, T, G);
    walk.end = share_start(w + 1, T, G);
    walk.next = 0;
    walk.mask = 0;
    walk.b0 = -64;
    walk.j = 64;
  }
  for (;;) {
    __syncthreads();  // walk initialised / every wavefront has read the previous piece
    if (tid < 64) flat_next_piece(a, walk, w, T, G);
    __syncthreads();
    const int b = __builtin_amdgcn_readfirstlane(walk.piece[0]);
    if (b < 0) return;
    const int L = __builtin_amdgcn_readfirstlane(walk.piece[1]);
    const int k0 = __builtin_amdgcn_readfirstlane(walk.piece[2]);
    const int k1 = __builtin_amdgcn_readfirstlane(walk.piece[3]);
    run_range<F, false, C>(a, smem, b, L, k0, k1, w + b, blockIdx.y);
  }
}

// ---------------------------------------------------------------- combine kernels
// Two wavefronts per (sequence, head), one per half of the 512 channels: lane
// owns channels 256 half + [4 lane, 4 lane + 4).  out = sum_s w_s o_s /
// sum_s w_s, w_s = exp(lse_s - max lse).  The weights are computed with one
// slot per lane (wavefront max and sum) and kept in LDS; the rows of eight
// slots are then in flight at a time, and rows of zero weight (empty pieces,
// lse = -inf, whose rows may hold anything) are never read.
// the balanced merge uses NC = 1 while its 8 H B wavefronts are at most
// two per SIMD (a few long sequences: many slots each, few rows)
constexpr int kCombineNarrowWaves = 2048;
constexpr int kCombineMaxSlots = 512;  // slots of one sequence: <= 64 splits or <= 512 balanced shares

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// Rows of one (sequence, head): wavefront `part` of the head's 8 / NC
// wavefronts owns channels [64 NC part, 64 NC (part + 1)), NC per lane; the
// weights are computed by every wavefront (the log-sum-exps are few and hit
// in L2).  The rows of 32 / NC slots are in flight at a time: NC = 1 keeps
// the loads of a few dozen slots in one round when the rows are few and the
// merge is latency-bound, NC = 4 streams 16-byte loads when they are many.
template <int NC>
__device__ __forceinline__ void combine_rows(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                                             int64_t first, int count, int64_t b, int H, int head, int part,
                                             float* __restrict__ wbuf, __bf16* __restrict__ out,
                                             float* __restrict__ lse_out) {
  using vec = float __attribute__((ext_vector_type(NC)));
  constexpr int U = 32 / NC;  // slots per round
  const int lane = threadIdx.x & 63;
  // a sequence has at most kCombineMaxSlots pieces; the clamp only keeps LDS
  // accesses in bounds for a workspace the decode did not write
  count = count < kCombineMaxSlots ? count : kCombineMaxSlots;
  const int ch = 64 * NC * part + NC * lane;
  const float* base = o_part + (first * H + head) * kDc + ch;
  // with one channel per lane and at most kPre slots, every row is loaded
  // before the weights are known, so the merge waits for memory once (rows
  // of zero weight are then read but not added)
  constexpr int kPre = NC == 1 ? 48 : 1;
  const bool pre = NC == 1 && count <= kPre;
  float xp[kPre];
  if (pre) {
#pragma unroll
    for (int j = 0; j < kPre; ++j) xp[j] = j < count ? base[(int64_t)j * H * kDc] : 0.0f;
  }
  // slot s's log-sum-exp in lane s % 64; the first 64 stay in a register
  const float ls0 = lane < count ? lse_part[(first + lane) * H + head] : -INFINITY;
  float M = ls0;
  for (int c0 = 64; c0 < count; c0 += 64) {
    const int s = c0 + lane;
    M = fmaxf(M, s < count ? lse_part[(first + s) * H + head] : -INFINITY);
  }
  M = wave_max(M);
  float W = 0.0f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < count; c0 += 64) {
      const int s = c0 + lane;
      const float ls = c0 == 0 ? ls0 : (s < count ? lse_part[(first + s) * H + head] : -INFINITY);
      const float w = s < count ? expf(ls - M) : 0.0f;
      if (s < count) wbuf[s] = w;
      W += w;
    }
    W = wave_sum(W);
  }
  vec acc = {};
  if (M != -INFINITY && pre) {
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const float w = j < count ? wbuf[j] : 0.0f;
      acc[0] += w > 0.0f ? w * xp[j] : 0.0f;
    }
  } else if (M != -INFINITY) {
    for (int s0 = 0; s0 < count; s0 += U) {
      float w[U];
      vec x[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        w[j] = s0 + j < count ? wbuf[s0 + j] : 0.0f;  // same address in every lane: a broadcast read
        x[j] = (vec){};
        if (w[j] > 0.0f) x[j] = *(const vec*)(base + (int64_t)(s0 + j) * H * kDc);  // uniform
      }
#pragma unroll
      for (int j = 0; j < U; ++j) acc += w[j] * x[j];
    }
  }
  const float inv = (M != -INFINITY) ? 1.0f / W : 0.0f;
  acc *= inv;
  __bf16* o = out + (b * H + head) * kDc + ch;
  if constexpr (NC == 4) {
    *(u32x2*)o = (u32x2){pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  } else {
    static_assert(NC == 1, "one or four channels per lane");
    *o = (__bf16)acc[0];
  }
  if (lse_out && part == 0 && lane == 0) lse_out[b * H + head] = (M != -INFINITY) ? M + logf(W) : -INFINITY;
}

// per-sequence splits: rows (b * S + s) * H + head
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                                                 int H, int S, __bf16* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ float wbuf[4][kCombineMaxSlots];
  const int b = blockIdx.y, wave = threadIdx.x >> 6;
  const int head = blockIdx.x * 2 + (wave >> 1);
  if (head >= H) return;
  combine_rows<4>(o_part, lse_part, (int64_t)b * S, S, b, H, head, wave & 1, wbuf[wave], out, lse_out);
}

// balanced partition: slots [meta[2b], meta[2b] + meta[2b + 1]) of sequence b
// (an empty sequence has count 0: output 0, lse -inf)
template <int NC>
__global__ __launch_bounds__(256) void k_combine_flat(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, const int* __restrict__ meta,
                                                      int H, __bf16* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ float wbuf[4][kCombineMaxSlots];
  constexpr int P = 8 / NC;  // wavefronts per head
  const int b = blockIdx.y, wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * 4 + wave;
  const int head = gw / P;
  if (head >= H) return;
  combine_rows<NC>(o_part, lse_part, meta[2 * b], meta[2 * b + 1], b, H, head, gw % P, wbuf[wave], out, lse_out);
}

// ---------------------------------------------------------------- launchers

// One head group per wavefront: two tiles and the LDS share of q, one
// workgroup per compute unit.  Channel split: the two tiles (the logit
// exchange reuses the tile being refilled) and each head group's shared
// weights; at C = 4 two workgroups share a compute unit (with the balanced
// kernel's 2112 static bytes, 80960 of the 81920 bytes each may hold).
constexpr size_t kDecodeLds = (2 * (size_t)kTile + 128 * kQRow) * sizeof(__bf16);  // 142336 bytes
template <int C> constexpr size_t decode_lds() {
  // channel split: two tiles and 4 KB of weights per head group (4 / C groups);
  // independent wavefronts: four V buffers and the merge record
  return C == 0 ? kIwLds : C > 1 ? 2 * (size_t)kTile * sizeof(__bf16) + 4096 * (4 / C) : kDecodeLds;
}

// The dynamic LDS size above 64 KB must be allowed once per kernel and device
// (bit d of `done` records device d; setting it twice is harmless).
template <typename K>
static hipError_t set_lds(K kernel, size_t bytes, std::atomic<unsigned long long>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_relaxed);
  return e;
}

// Kernel variant by rows per sequence for the quantized formats:
// independent wavefronts at <= 16 rows (0), all 4 wavefronts on one group of
// 17..32 rows (two workgroups per compute unit),
// 2 wavefronts per group for 33..64 rows, else one head group per wavefront
// (the unquantized baseline always uses the latter).  On 8 x 131072 C4R4
// tokens, balanced: 16 heads 0.222 -> 0.167 ms (channel split) -> 0.11 ms
// (independent wavefronts), 64 heads 0.309 -> 0.27 ms.
static int channel_split(int fmt, int rows) {
  if (fmt == kBF16) return 1;
  return rows <= 16 ? 0 : rows <= 32 ? 4 : rows <= 64 ? 2 : 1;
}

int workgroups_per_cu(int fmt, int rows) { return channel_split(fmt, rows) == 4 ? 2 : 1; }

// Head chunks of a launch (grid dimension): s_q * chunk_heads rows each.
static int head_chunks(const DecodeArgs& a) { return (a.qheads + a.chunk_heads - 1) / a.chunk_heads; }

template <int F, bool D, int C>
static hipError_t launch_one(const DecodeArgs& a, int batch, hipStream_t stream) {
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t e = set_lds(k_decode<F, D, C>, decode_lds<C>(), attr_done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode<F, D, C>), dim3(a.num_splits, batch, head_chunks(a)), dim3(decode_threads<C>()),
                     decode_lds<C>(),
                     stream, a);
  return hipGetLastError();
}

template <int F, int C>
static hipError_t launch_flat_one(const DecodeArgs& a, int groups, hipStream_t stream) {
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t e = set_lds(k_decode_flat<F, C>, decode_lds<C>(), attr_done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode_flat<F, C>), dim3(groups, head_chunks(a)), dim3(decode_threads<C>()), decode_lds<C>(),
                     stream, a);
  return hipGetLastError();
}

template <int F, int C>
static hipError_t launch_split(bool direct, const DecodeArgs& a, int batch, hipStream_t stream) {
  return direct ? launch_one<F, true, C>(a, batch, stream) : launch_one<F, false, C>(a, batch, stream);
}

hipError_t launch_decode(int fmt, bool direct, const DecodeArgs& a, int batch, hipStream_t stream) {
  const int c = channel_split(fmt, a.s_q * a.chunk_heads);
  if (fmt == kC4R4)
    return c == 0 ? launch_split<kC4R4, 0>(direct, a, batch, stream)
           : c == 4 ? launch_split<kC4R4, 4>(direct, a, batch, stream)
           : c == 2 ? launch_split<kC4R4, 2>(direct, a, batch, stream)
                    : launch_split<kC4R4, 1>(direct, a, batch, stream);
  if (fmt == kC2R4)
    return c == 0 ? launch_split<kC2R4, 0>(direct, a, batch, stream)
           : c == 4 ? launch_split<kC2R4, 4>(direct, a, batch, stream)
           : c == 2 ? launch_split<kC2R4, 2>(direct, a, batch, stream)
                    : launch_split<kC2R4, 1>(direct, a, batch, stream);
  return launch_split<kBF16, 1>(direct, a, batch, stream);
}

hipError_t launch_decode_flat(int fmt, const DecodeArgs& a, int groups, hipStream_t stream) {
  const int c = channel_split(fmt, a.s_q * a.chunk_heads);
  if (fmt == kC4R4)
    return c == 0 ? launch_flat_one<kC4R4, 0>(a, groups, stream)
           : c == 4 ? launch_flat_one<kC4R4, 4>(a, groups, stream)
           : c == 2 ? launch_flat_one<kC4R4, 2>(a, groups, stream)
                    : launch_flat_one<kC4R4, 1>(a, groups, stream);
  if (fmt == kC2R4)
    return c == 0 ? launch_flat_one<kC2R4, 0>(a, groups, stream)
           : c == 4 ? launch_flat_one<kC2R4, 4>(a, groups, stream)
           : c == 2 ? launch_flat_one<kC2R4, 2>(a, groups, stream)
                    : launch_flat_one<kC2R4, 1>(a, groups, stream);
  return launch_flat_one<kBF16, 1>(a, groups, stream);
}

hipError_t launch_combine(const float* o_part, const float* lse_part, int batch, int heads, int splits,
                          __bf16* out, float* lse_out, hipStream_t stream) {
  hipLaunchKernelGGL(k_combine, dim3((heads + 1) / 2, batch), dim3(256), 0, stream, o_part, lse_part, heads, splits,
                     out, lse_out);
  return hipGetLastError();
}

hipError_t launch_combine_flat(const float* o_part, const float* lse_part, const int* meta, int batch, int heads,
                               __bf16* out, float* lse_out, hipStream_t stream) {
  if (8ll * heads * batch <= kCombineNarrowWaves)
    hipLaunchKernelGGL(k_combine_flat<1>, dim3(2 * heads, batch), dim3(256), 0, stream, o_part, lse_part, meta,
                       heads, out, lse_out);
  else
    hipLaunchKernelGGL(k_combine_flat<4>, dim3((heads + 1) / 2, batch), dim3(256), 0, stream, o_part, lse_part,
                       meta, heads, out, lse_out);
  return hipGetLastError();
}

}  // namespace mla
