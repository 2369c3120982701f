// Grouped GEMM on bf16 MFMA for the expert projections (page "MoE: how
// sparse activation saves compute", section 3.1: F(u) = W_down act(W_gate u,
// W_up u); section 3.6: expert i works on its own [L_i, d] block of rows).
//
//   C_g[r, n] = sum_k A[arow(g, r), k] * B_g[n, k]      (both operands K-contiguous)
//
// One 256x256 output tile per 512-thread workgroup: 8 waves, two per SIMD,
// each 128x64 on v_mfma_f32_32x32x16_bf16 (8 accumulator blocks, 223 VGPRs
// so two waves fit a SIMD).  The second wave on a SIMD issues MFMAs while its
// sibling waits on a load issue or the barrier.  K advances 64 at a time.
// A (the activations, mostly L2 hits) is double-buffered and B (the weights,
// streamed) sits in a ring of three 32 KiB LDS stages -- 160 KiB in all --
// filled by direct global->LDS buffer loads (no VGPR staging); A
// rows are gathered through the dispatch permutation by those loads, so the
// expert-sorted copy of the activations is never written.  Per k-step: three
// 8-MFMA sub-steps, each overlapping the next sub-step's fragment reads, one
// barrier, and a fourth sub-step that overlaps the next stage's first reads.
// The loads are spread over the k-step (B two stages ahead in sub-steps 0-1,
// A one stage ahead in sub-step 3) so the address unit works alongside the
// MFMAs instead of in one burst after the barrier.
// Tiles are found on the device from the per-group m-tile prefix and spread
// over the XCDs in contiguous ranges; surplus workgroups exit, so the host
// never waits for the routing result.  In an expert's last, partly filled
// m-tile a wave whose last 32-row block holds no row skips that block's
// fragment reads and MFMAs (a second copy of the main loop).
//
// Epilogues: EP_GLU pairs 128 gate columns with the matching 128 up columns in
// one tile and writes act(gate, up) as bf16 (the hidden of a SwiGLU or
// SiTU-GLU expert), EP_GLU_SAVE also the gate and up sums themselves (bf16,
// kept for the backward); EP_F32 stores the fp32 product through LDS so each store
// writes a whole output row, and handles any column count (the router logits
// have N columns); EP_BF16 stores the rounded product; EP_ADD_BF16 adds two
// fp32 matrices before rounding (the latent layer's shared-expert outputs).
// The bf16 epilogues store 4 columns at a time: their column counts (h, d, l)
// are multiples of 128.
//
// Transposed B (the experts' backward: dH against W_down, dx against
// [W_gate ; W_up], read as stored): the B stage holds [64 k][256 n] rows
// filled by the same direct loads (each k row is one contiguous 512-byte run
// of the weights), and each B fragment is two ds_read_b64_tr_b16, which hand
// every lane four consecutive k of one column.
//
// MXFP4 weights (routed experts, EP_GLU and EP_F32): 8 KiB B stages of
// 32-byte rows of packed E2M1 pairs, one direct load per wave per stage; the
// tile's E8M0 scales go to LDS in 4096-k chunks (256 rows x 128 bytes), the
// first ahead of stage 0 and each next one a k-step into the chunk before it
// (two tables in turn), and each fragment's 8 codes are widened with their
// block's scale by v_cvt_scalef32_pk_bf16_fp4 (exact in bf16).
//
// FP8 weights (routed experts, EP_GLU and EP_F32): B holds OCP E4M3 codes,
// one 64-byte row per weight row and k-step in a 16 KiB stage, 16-byte
// chunk c of row r at chunk c ^ ((r >> 2) & 3); each fragment read takes 8
// codes and widens them exactly to bf16, and the per-row scales multiply the
// fp32 sums in the epilogue.
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;  // 8 waves: two per SIMD
constexpr int kBBytes = BN * BK * 2;   // 32 KiB per B stage
constexpr int kMSuper = 8;                       // m-tiles per scheduling group

// Byte offset of 16-byte chunk c of row r inside one [256][64] bf16 tile.
// The chunk is XOR-swizzled with row bits 1-3: two 128-byte rows share the
// 64 banks, so the 16 rows of a fragment read's lane phase land on 16
// distinct 16-byte bank groups (bits 0-2 left rows r and r + 8 on the same
// banks, a 2-way conflict on every fragment read).
__device__ __forceinline__ uint32_t swz(int r, int c) {
  return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
}

__device__ __forceinline__ bf16x8 lds_frag(const char *tile, int r, int c) {
  return *reinterpret_cast<const bf16x8 *>(tile + swz(r, c));
}

// FP8 B stage: the 8 codes of k-step quarter kq (0..7) of row r, widened.
__device__ __forceinline__ bf16x8 lds_frag8(const char *tile, int r, int kq) {
  const int c = kq >> 1;
  const uint2 raw = *reinterpret_cast<const uint2 *>(
      tile + r * 64 + ((c ^ ((r >> 2) & 3)) << 4) + 8 * (kq & 1));
  return e4m3x8_to_bf16x8(raw.x, raw.y);
}

// MXFP4 B stage: 32-byte rows of packed E2M1 (64 k per row and k-step),
// 16-byte chunk c of row r at chunk c ^ ((r >> 3) & 1); four codes of the
// fragment's eight (k-step quarter kq of row r) are one u32.
__device__ __forceinline__ uint32_t lds_frag4(const char *tile, int r, int kq) {
  const int c = kq >> 2;
  return *reinterpret_cast<const uint32_t *>(tile + r * 32 + ((c ^ ((r >> 3) & 1)) << 4) +
                                             4 * (kq & 3));
}

// BM = 256 (waves 128x64) or 192 (waves 96x64, for experts with few rows).
// MX4: B holds MXFP4 weights (packed E2M1 + one E8M0 scale byte per 32 k).
template <int EPI, int BM, bool FP8 = false, bool KSEG = false, bool BT = false,
          bool MX4 = false>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmArgs a) {
  static_assert(!FP8 || EPI == EP_GLU || EPI == EP_F32, "fp8 weights: routed experts only");
  static_assert(!MX4 || ((EPI == EP_GLU || EPI == EP_F32) && !FP8 && !KSEG && !BT),
                "MXFP4 weights: routed experts only");
  static_assert(!KSEG || (EPI == EP_F32 && !FP8), "k segments: fp32 weight gradients");
  static_assert(!FP8 || EPI != EP_GLU_SAVE, "saved gate/up sums: bf16 weights");
  static_assert(!BT || (!FP8 && !KSEG && EPI != EP_GLU && EPI != EP_GU && EPI != EP_GLU_SAVE),
                "transposed B: bf16, one B row per output column");
  constexpr int ES = FP8 ? 1 : 2;          // bytes per B element (MX4: half a byte)
  // B stage stride: MX4 stages are 8 KiB, and the tile's scale table
  // follows the three stages.
  constexpr int kBStage = MX4 ? 8192 : kBBytes;
  // Two 32 KiB scale tables follow: each holds one 4096-k chunk of the
  // tile's E8M0 scales ([256 rows][128 bytes]); chunk c sits in table c & 1.
  constexpr int kScaleOff = 3 * 8192;
  constexpr int kTab = 256 * 128;
  constexpr int MI = BM / 64;              // 32-row A blocks per wave
  constexpr int kABytes = BM * BK * 2;     // 32 or 24 KiB per A stage
  // A (activations, L2-resident) double-buffered; B (weights, streamed) in a
  // ring of three so its loads get two k-steps of cover: 160 / 144 KiB.
  __shared__ __attribute__((aligned(16))) char smem[2 * kABytes + 3 * kBBytes];
  // 256-row tiles (many rows per expert: each weight chunk serves 8 m-tiles
  // on the XCD, each activation chunk 4 n-tiles) take the rings the other way
  // round for bf16 K-contiguous B: A in three buffers, so that the gathered
  // rows get two k-steps of cover, B in two (Mixtral prefill gate/up 6.04 ->
  // 5.99 ms, Switch 2.06 -> 2.03 ms).  192-row tiles keep B's three: there
  // (LatentMoE, few rows per expert) the weights stream from HBM and need
  // the cover (swapped: 8.09 -> 8.56 ms).
  constexpr bool kASwap = BM == 256 && !FP8 && !MX4 && !BT && !KSEG;
  constexpr int kBBase = (kASwap ? 3 : 2) * kABytes;  // B stages start here
  static_assert(!kASwap || 3 * kABytes + 2 * kBBytes <= 2 * kABytes + 3 * kBBytes, "LDS");

  // ---- which tile: XCD-aware remap (block i runs on XCD i % 8: each XCD
  // takes one contiguous eighth of the real tiles), then (group, m-super, n,
  // m) order so the tiles running together on one XCD share A and B rows.
  const int glu = (EPI == EP_GLU || EPI == EP_GU || EPI == EP_GLU_SAVE);
  const int64_t NT = glu ? (a.ncols + 127) / 128 : (a.ncols + BN - 1) / BN;
  const int64_t real_tiles = (a.mode == GM_DENSE)
                                 ? (int64_t)a.G * ((a.M_dense + BM - 1) / BM) * NT
                                 : (int64_t)a.tile_start[a.G] * NT;
  // The grid is an upper bound on the tile count, so it can exceed 8 x per;
  // the remap is one-to-one only on blocks 0 .. 8 x per - 1, and any block
  // past that would land on a tile of the next XCD's range a second time.
  const int64_t bid = blockIdx.x;
  const int64_t per = (real_tiles + 7) >> 3;
  if ((bid >> 3) >= per) return;
  const int64_t L = (bid & 7) * per + (bid >> 3);
  if (L >= real_tiles) return;

  int g;
  int64_t local, MTg, Mg;
  if (a.mode == GM_DENSE) {
    const int64_t MT = (a.M_dense + BM - 1) / BM;
    g = (int)(L / (MT * NT));
    local = L - (int64_t)g * MT * NT;
    MTg = MT;
    Mg = a.M_dense;
  } else {
    int lo = 0, hi = a.G;  // largest g with tile_start[g] * NT <= L
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)a.tile_start[mid] * NT <= L) lo = mid; else hi = mid;
    }
    g = lo;
    local = L - (int64_t)a.tile_start[g] * NT;
    MTg = a.tile_start[g + 1] - a.tile_start[g];
    Mg = a.kept_offsets[g + 1] - a.kept_offsets[g];
  }
  const int64_t ms = local / (kMSuper * NT);
  const int64_t rem = local - ms * kMSuper * NT;
  const int64_t msz = (MTg - ms * kMSuper) < kMSuper ? (MTg - ms * kMSuper) : kMSuper;
  const int64_t n_tile = rem / msz;
  const int64_t m_tile = ms * kMSuper + (rem - n_tile * msz);
  const int64_t m0 = m_tile * BM;
  const int mrows = (int)((Mg - m0) < BM ? (Mg - m0) : BM);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lc = tid & 7;    // loader chunk
  const int lr = tid >> 3;   // loader base row (0..63)

  // ---- loader offsets (bytes), fixed over the K loop.
  const int64_t seg0 = (a.mode == GM_DENSE) ? 0 : a.kept_offsets[g];
  // Per-wave arrays are sized for the largest MI (4) and used up to MI: host
  // compilation drops the launch stub of a kernel template whose local arrays
  // have a template-dependent size.
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = lr + 64 * i;
    const int64_t rr = m0 + (r < mrows ? r : mrows - 1);
    int64_t arow;
    if (a.mode == GM_GATHER) arow = a.perm[a.offsets[g] + rr] / a.kslots;
    else if (a.mode == GM_SEGMENT) arow = seg0 + rr;
    else arow = (int64_t)g * a.a_group_rows + rr;
    const int pc = lc ^ ((r >> 1) & 7);  // the chunk this lane's LDS slot holds
    aoff[i] = (uint32_t)(arow * a.lda * 2) + (uint32_t)(pc << 4);
  }
  // B rows: bf16, instruction i fills rows 64i + tid/8 (8 lanes a row);
  // fp8, instruction i (0, 1) fills rows 128i + tid/4 (4 lanes a row).
  // Transposed B: the stage is [64 k][256 n] (512-byte rows, 16-byte chunk c
  // of row k at chunk c ^ 4 (k & 3)); instruction i of wave w fills rows
  // 2 (8i + w) and 2 (8i + w) + 1, lane l row + l / 32, chunk l % 32.
  // MXFP4: one instruction per wave fills rows 32 w .. 32 w + 31 (two lanes
  // a row), waves 0-3 the gate rows and 4-7 the up rows of a GLU tile.
#pragma unroll
  for (int i = 0; i < (FP8 ? 2 : 4); ++i) {
    if constexpr (MX4) {
      if (i == 0) {
        const int r = tid >> 1;
        const int pc = (tid & 1) ^ ((r >> 3) & 1);
        int64_t brow;
        if (glu) {
          const int64_t n = n_tile * 128 + (r & 127);
          brow = n < a.ncols ? n : a.ncols - 1;
        } else {
          const int64_t n = n_tile * BN + r;
          brow = n < a.ncols ? n : a.ncols - 1;
        }
        boff[0] = (uint32_t)(brow * (a.K / 2)) + (uint32_t)(pc << 4);
      }
      continue;
    }
    if constexpr (BT) {
      const int kr = 2 * (8 * i + wave) + (lane >> 5);
      const int c = (lane & 31) ^ ((kr & 3) << 2);
      int64_t n = n_tile * BN + 8 * c;
      if (n + 8 > a.ncols) n = a.ncols - 8;
      boff[i] = (uint32_t)((kr * a.ldbt + n) * 2);
      continue;
    }
    const int r = FP8 ? (tid >> 2) + 128 * i : lr + 64 * i;
    const int pc = FP8 ? ((tid & 3) ^ ((r >> 2) & 3)) : (lc ^ ((r >> 1) & 7));
    int64_t brow;
    if (glu) {
      const int64_t n = n_tile * 128 + (r & 127);
      brow = n < a.ncols ? n : a.ncols - 1;
    } else {
      const int64_t n = n_tile * BN + r;
      brow = n < a.ncols ? n : a.ncols - 1;
    }
    boff[i] = (uint32_t)(brow * (KSEG ? a.ldb : a.K) * ES) + (uint32_t)(pc << 4);
  }
  const char *Bg = static_cast<const char *>(a.B) + (MX4 ? (int64_t)g * a.strideB / 2
                                                             : (int64_t)g * a.strideB * ES);
  const char *Ug = (glu || (BT && a.ksplit > 0))
                       ? static_cast<const char *>(a.B2) +
                             (MX4 ? (int64_t)g * a.strideB / 2 : (int64_t)g * a.strideB * ES)
                       : Bg;
  const uint32_t bbytes =
      BT    ? (uint32_t)((int64_t)(a.ksplit > 0 ? a.ksplit : a.K) * a.ldbt * 2)
      : MX4 ? (uint32_t)((int64_t)a.ncols * a.K / 2)
            : (uint32_t)((int64_t)a.ncols * (KSEG ? a.ldb : a.K) * ES);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, bbytes);
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(Ug, bbytes);

  // Direct global -> LDS loads: instruction i of wave w fills the 1 KiB of
  // rows 64i + 8w .. +7 and lane l lands at byte 16 l of it.
  typedef __attribute__((address_space(3))) void *lds_ptr_t;
  // K segments: this group's k range starts at kbase.
  const int kbase = KSEG ? (a.kseg != nullptr ? a.kseg[g] : g * a.kchunk) : 0;
  auto aload_rows = [&](int k0, int buf, int i0, int i1) {
    const uint32_t so = (uint32_t)(kbase + k0) * 2;
    char *ta = smem + buf * kABytes;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      if (i >= i0 && i < i1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(ta + (64 * i + 8 * wave) * 128),
                                                 16, aoff[i], so, 0, 0);
  };
  auto aload = [&](int k0, int buf) { aload_rows(k0, buf, 0, MI); };
  auto bload = [&](int k0, int buf, int half) {
    const uint32_t so = (uint32_t)(kbase + k0) * ES;
    char *tb = smem + kBBase + buf * kBStage;
    if constexpr (MX4) {
      if (half == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds((glu && wave >= 4) ? ru : rb,
                                                 (lds_ptr_t)(tb + wave * 1024), 16, boff[0],
                                                 (uint32_t)k0 / 2, 0, 0);
    } else if constexpr (BT) {
      // A k-step lies wholly in B or in B2 (ksplit is a multiple of BK).
      const bool second = a.ksplit > 0 && k0 >= a.ksplit;
      const uint32_t sot = (uint32_t)((int64_t)(second ? k0 - a.ksplit : k0) * a.ldbt * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = 2 * half + j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? ru : rb,
                                                 (lds_ptr_t)(tb + (8 * i + wave) * 1024), 16,
                                                 boff[i], sot, 0, 0);
      }
    } else if constexpr (FP8) {
      // GLU: rows 0-127 gate, 128-255 up.
      __builtin_amdgcn_raw_ptr_buffer_load_lds((glu && half) ? ru : rb,
                                               (lds_ptr_t)(tb + (128 * half + 16 * wave) * 64),
                                               16, boff[half], so, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = 2 * half + j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds((glu && i >= 2) ? ru : rb,
                                                 (lds_ptr_t)(tb + (64 * i + 8 * wave) * 128), 16,
                                                 boff[i], so, 0, 0);
      }
    }
  };

  // Per-wave fragment rows.
  int arow_l[4], brow_l[2];
#pragma unroll
  for (int i = 0; i < MI; ++i) arow_l[i] = wm * (BM / 2) + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    brow_l[j] = glu ? (wn * 32 + j * 128 + (lane & 31)) : (wn * 64 + j * 32 + (lane & 31));
  const int khalf = lane >> 5;
  // Transposed B: each fragment (8 consecutive k of one column n) is two
  // transposing LDS reads of 4 k each.  Within a 16-lane group (g16 = lane
  // / 16, r = lane % 16) lane r addresses row 8 (g16 / 2) + r / 4 (+ 4 for
  // the second read, + 16 per sub-step) at column n0 + 4 (r % 4), and lane
  // 4q + e receives element e of the rows addressed by lanes q, q + 4,
  // q + 8, q + 12: the four k of column n0 + 4q + e.
  int bt_off[2];
  if constexpr (BT) {
    const int g16 = lane >> 4, r = lane & 15;
    const int kr = 8 * (g16 >> 1) + (r >> 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn * 64 + j * 32 + 16 * (g16 & 1) + 4 * (r & 3);
      bt_off[j] = kr * 512 + (((n >> 3) ^ ((kr & 3) << 2)) << 4) + (n & 7) * 2;
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 fa[4], fb[2], na[4], nb[2];
  // The main loop, for the first M of the wave's MI 32-row A blocks: a wave
  // whose last block lies wholly past the tile's rows (an expert's last,
  // partly filled m-tile) skips that block's fragment reads and MFMAs.
  auto main_loop = [&](auto mconst) {
  constexpr int M = decltype(mconst)::value;
  auto read_frags = [&](int kt, int ks, bf16x8 (&xa)[4], bf16x8 (&xb)[2]) {
    const char *ta = smem + (kASwap ? kt % 3 : kt & 1) * kABytes;
    const char *tb = smem + kBBase + (kASwap ? kt & 1 : kt % 3) * kBStage;
    const int c = ks * 2 + khalf;
#pragma unroll
    for (int i = 0; i < M; ++i) xa[i] = lds_frag(ta, arow_l[i], c);
    if constexpr (MX4) {
      // 8 codes of quarter c (32-k block kt * 2 + ks / 2) times the block's
      // scale from the chunk's table.
      const unsigned char *sct = reinterpret_cast<const unsigned char *>(
          smem + 2 * kABytes + kScaleOff + ((kt >> 6) & 1) * kTab);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float sc = e8m0_to_f32(sct[brow_l[j] * 128 + (kt & 63) * 2 + (ks >> 1)]);
        xb[j] = e2m1x8_to_bf16x8(lds_frag4(tb, brow_l[j], c), sc);
      }
    } else if constexpr (BT) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s *lds_v4s_t;
      typedef short v8s __attribute__((ext_vector_type(8)));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char *p0 = tb + bt_off[j] + ks * 16 * 512;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t)(p0));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t)(p0 + 4 * 512));
        const v8s w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        xb[j] = __builtin_bit_cast(bf16x8, w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        xb[j] = FP8 ? lds_frag8(tb, brow_l[j], c) : lds_frag(tb, brow_l[j], c);
    }
  };
  auto mfma16 = [&](const bf16x8 (&xa)[4], const bf16x8 (&xb)[2]) {
#pragma unroll
    for (int i = 0; i < M; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb[j], xa[i], acc[i][j], 0, 0, 0);
  };
  auto copy_frags = [&]() {
#pragma unroll
    for (int i = 0; i < M; ++i) fa[i] = na[i];
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = nb[j];
  };

  // A sub-step is one fenced scheduling region: the fragment reads for the
  // next sub-step (and any loads) interleaved with this sub-step's 8 MFMAs.
#define MOE_SUBSTEP(READ_STMT, EXTRA_STMT, EXTRA_MASK, EXTRA_N)          \
  do {                                                                  \
    READ_STMT;                                                          \
    EXTRA_STMT;                                                         \
    mfma16(fa, fb);                                                     \
    _Pragma("unroll") for (int i_ = 0; i_ < M; ++i_) {                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                \
      __builtin_amdgcn_sched_group_barrier(EXTRA_MASK, EXTRA_N, 0);     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                \
    }                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                  \
    copy_frags();                                                       \
  } while (0)
#define MOE_WAIT_LOADS() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")

  // K >= 128, so KT >= 2.  Stage s: A in buffer s & 1, B in buffer s % 3.
  // Loads are spread over the k-step so the address unit works alongside the
  // MFMAs: B(kt+2) during sub-steps 0-1 of step kt (buffer (kt+2) % 3 was
  // released by the barrier ending step kt-1), A(kt+2) during sub-step 3
  // after step kt's barrier.  Before a barrier only B(kt+2) may still fly.
  const int KT = (KSEG ? (a.kseg != nullptr ? a.kseg[g + 1] - a.kseg[g] : a.kchunk) : a.K) / BK;
  // MXFP4: scale table of 4096-k chunk c into table buf, 16 dword loads per
  // wave (every wave and every chunk the same count, for the in-order load
  // counting); a short last chunk repeats its last dword.
  auto load_table = [&](int c, int buf) {
    const int kc = a.K / 32 - 128 * c;  // this chunk's scale bytes per row
    const int rdw = (kc < 128 ? kc : 128) / 4;
    const int64_t sbytes = (int64_t)a.ncols * (a.K / 32);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(reinterpret_cast<const unsigned char *>(a.bscale) + g * sbytes,
                  (uint32_t)sbytes);
    const __amdgpu_buffer_rsrc_t rs2 =
        glu ? make_rsrc(reinterpret_cast<const unsigned char *>(a.bscale2) + g * sbytes,
                        (uint32_t)sbytes)
            : rs;
    char *st = smem + 2 * kABytes + kScaleOff + buf * kTab;
#pragma unroll
    for (int q = 0; q < kTab / (4 * kThreads); ++q) {
      const int f = q * kThreads + tid;
      const int r = f >> 5, dw0 = f & 31;
      const int dw = dw0 < rdw ? dw0 : rdw - 1;
      int64_t brow;
      if (glu) {
        const int64_t n = n_tile * 128 + (r & 127);
        brow = n < a.ncols ? n : a.ncols - 1;
      } else {
        const int64_t n = n_tile * BN + r;
        brow = n < a.ncols ? n : a.ncols - 1;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          (glu && r >= 128) ? rs2 : rs, (lds_ptr_t)(st + q * kThreads * 4 + wave * 256), 4,
          (uint32_t)(brow * (a.K / 32) + 128 * c + 4 * dw), 0, 0, 0);
    }
  };
  if constexpr (MX4) load_table(0, 0);  // ahead of stage 0: its wait covers it
  aload(0, 0);
  bload(0, 0, 0);
  bload(0, 0, 1);
  aload(BK, 1);
  bload(BK, 1, 0);
  bload(BK, 1, 1);
  // stage 0 landed: stage 1's MI A loads and 4 (fp8: 2, MXFP4: 1) B loads
  // may fly
  if constexpr (MX4 && MI == 4) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else if constexpr (MX4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (MI == 4 && !FP8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (MI == 3 && !FP8) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  else if constexpr (MI == 4) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  barrier_keep_loads();
  read_frags(0, 0, fa, fb);
  if constexpr (kASwap) {
    // A(kt+2) during sub-steps 0-1 of step kt (buffer (kt+2) % 3 was
    // released by the barrier ending step kt-1), B(kt+2) after step kt's
    // barrier; before a barrier only A(kt+2) may still fly.
    for (int kt = 0; kt + 2 < KT; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
      MOE_SUBSTEP(read_frags(kt, 1, na, nb), aload_rows((kt + 2) * BK, (kt + 2) % 3, 0, (MI + 1) / 2),
                  0x020, 1);
      MOE_SUBSTEP(read_frags(kt, 2, na, nb), aload_rows((kt + 2) * BK, (kt + 2) % 3, (MI + 1) / 2, MI),
                  0x020, 1);
      MOE_SUBSTEP(read_frags(kt, 3, na, nb), (void)0, 0x000, 0);
      if constexpr (MI == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
      barrier_keep_loads();
      __builtin_amdgcn_sched_barrier(0);
      MOE_SUBSTEP(read_frags(kt + 1, 0, na, nb),
                  (bload((kt + 2) * BK, kt & 1, 0), bload((kt + 2) * BK, kt & 1, 1)), 0x020, 1);
    }
  } else
  for (int kt = 0; kt + 2 < KT; ++kt) {
    __builtin_amdgcn_sched_barrier(0);
    MOE_SUBSTEP(read_frags(kt, 1, na, nb), bload((kt + 2) * BK, (kt + 2) % 3, 0), 0x020, 1);
    // MXFP4, K > 4096: the next chunk's scales, one k-step into this chunk
    // (table (c + 1) & 1 last served chunk c - 1, finished two barriers ago).
    const bool tab = MX4 && (kt & 63) == 1 && (kt >> 6) < ((KT - 1) >> 6);
    if constexpr (MX4) {
      if (tab) load_table((kt >> 6) + 1, ((kt >> 6) + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    MOE_SUBSTEP(read_frags(kt, 2, na, nb), bload((kt + 2) * BK, (kt + 2) % 3, 1), 0x020, 1);
    MOE_SUBSTEP(read_frags(kt, 3, na, nb), (void)0, 0x000, 0);
    // stage kt+1 landed; only B(kt+2) may still fly (and a chunk's table
    // loads issued after it)
    if constexpr (MX4) {
      if (tab) asm volatile("s_waitcnt vmcnt(17)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    } else if constexpr (FP8) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    barrier_keep_loads();
    __builtin_amdgcn_sched_barrier(0);
    MOE_SUBSTEP(read_frags(kt + 1, 0, na, nb), aload((kt + 2) * BK, kt & 1), 0x020, 1);
  }
  {
    const int kt = KT - 2;
    __builtin_amdgcn_sched_barrier(0);
    MOE_SUBSTEP(read_frags(kt, 1, na, nb), (void)0, 0x000, 0);
    MOE_SUBSTEP(read_frags(kt, 2, na, nb), (void)0, 0x000, 0);
    MOE_SUBSTEP(read_frags(kt, 3, na, nb), (void)0, 0x000, 0);
    MOE_WAIT_LOADS();
    barrier_keep_loads();
    __builtin_amdgcn_sched_barrier(0);
    MOE_SUBSTEP(read_frags(kt + 1, 0, na, nb), (void)0, 0x000, 0);
    __builtin_amdgcn_sched_barrier(0);
    MOE_SUBSTEP(read_frags(kt + 1, 1, na, nb), (void)0, 0x000, 0);
    MOE_SUBSTEP(read_frags(kt + 1, 2, na, nb), (void)0, 0x000, 0);
    MOE_SUBSTEP(read_frags(kt + 1, 3, na, nb), (void)0, 0x000, 0);
    mfma16(fa, fb);
  }
  };  // main_loop
  if (mrows - wm * (BM / 2) > (MI - 1) * 32) main_loop(std::integral_constant<int, MI>{});
  else main_loop(std::integral_constant<int, MI - 1>{});
#undef MOE_WAIT_LOADS
#undef MOE_SUBSTEP

  // FP8: the scales of this lane's output columns (the weight rows), for
  // block j and column group q: 4 columns from n_tile*BN + wn*64 + 32j + 8q
  // + 4*khalf (GLU: j = 0 the gate rows, j = 1 the up rows of the columns
  // n_tile*128 + wn*32 + 8q + 4*khalf).  Columns past the end read a valid
  // row and are never stored.
  f32x4 bsc[2][4];
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float *S = (glu && j) ? a.bscale2 : a.bscale;
        const int64_t c0 = glu ? n_tile * 128 + wn * 32 + 8 * q + 4 * khalf
                               : n_tile * BN + wn * 64 + j * 32 + 8 * q + 4 * khalf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t c = c0 + e < a.ncols ? c0 + e : a.ncols - 1;
          bsc[j][q][e] = S[(int64_t)g * a.ncols + c];
        }
      }
  }

  if constexpr (EPI == EP_F32) {
    // fp32 tile through LDS, the rows of one wm at a time, so that each store
    // instruction writes one whole 1 KiB output row (the register layout
    // would write 32-byte pieces of 32 rows).  Row pitch padded by 16 bytes.
    constexpr int kRows = BM / 2;
    constexpr int kPitch = BN * 4 + 16;
    static_assert(kRows * kPitch <= 2 * kABytes + 3 * kBBytes, "staging exceeds LDS");
    __syncthreads();  // every wave has finished reading the operand stages
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int rl = i * 32 + (lane & 31);
              const int c = wn * 64 + j * 32 + 8 * q + 4 * khalf;
              f32x4 v = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                              acc[i][j][4 * q + 3]};
              if constexpr (FP8) v *= bsc[j][q];
              *reinterpret_cast<f32x4 *>(smem + rl * kPitch + c * 4) = v;
            }
      }
      __syncthreads();
      const int64_t col = n_tile * BN + 4 * lane;
      for (int rl = wave; rl < kRows; rl += kThreads / 64) {
        const int r = half * kRows + rl;
        if (r >= mrows || col >= a.ncols) continue;
        const int64_t orow = (a.mode == GM_DENSE) ? (int64_t)g * a.out_group_stride + m0 + r
                                                  : seg0 + m0 + r;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(smem + rl * kPitch + 16 * lane);
        float *dst = reinterpret_cast<float *>(a.out) + orow * a.ldo + col;
        if (col + 4 <= a.ncols) {
          *reinterpret_cast<f32x4 *>(dst) = v;
        } else {
          for (int e = 0; e < (int)(a.ncols - col); ++e) dst[e] = v[e];
        }
      }
      __syncthreads();
    }
    return;
  }

  // ---- epilogue.  Lane holds, for A block i and B block j, output row
  // wm*128 + i*32 + lane%32 and columns 8q + 4*(lane/32) + {0..3}, q = 0..3,
  // of the wave's 32-column block j (GLU: j = 0 gate, j = 1 up).
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = wm * (BM / 2) + i * 32 + (lane & 31);
    if (r >= mrows) continue;
    const int64_t orow = (a.mode == GM_DENSE) ? (int64_t)g * a.out_group_stride + m0 + r
                                              : seg0 + m0 + r;
    if constexpr (EPI == EP_GU) {
      // Gate and up sums, each rounded to bf16.
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n_tile * 128 + wn * 32 + 8 * q + 4 * khalf;
        if (col >= a.ncols) continue;
        uint2 pg, pu;
        pg.x = pack_bf16x2_hw(acc[i][0][4 * q], acc[i][0][4 * q + 1]);
        pg.y = pack_bf16x2_hw(acc[i][0][4 * q + 2], acc[i][0][4 * q + 3]);
        pu.x = pack_bf16x2_hw(acc[i][1][4 * q], acc[i][1][4 * q + 1]);
        pu.y = pack_bf16x2_hw(acc[i][1][4 * q + 2], acc[i][1][4 * q + 3]);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + orow * a.ldo + col) = pg;
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out2) + orow * a.ldo + col) =
            pu;
      }
    } else if constexpr (EPI == EP_GLU || EPI == EP_GLU_SAVE) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n_tile * 128 + wn * 32 + 8 * q + 4 * khalf;
        if (col >= a.ncols) continue;
        if constexpr (EPI == EP_GLU_SAVE) {
          // G and U, each rounded to bf16, as the backward's recompute would.
          uint2 pg, pu;
          pg.x = pack_bf16x2_hw(acc[i][0][4 * q], acc[i][0][4 * q + 1]);
          pg.y = pack_bf16x2_hw(acc[i][0][4 * q + 2], acc[i][0][4 * q + 3]);
          pu.x = pack_bf16x2_hw(acc[i][1][4 * q], acc[i][1][4 * q + 1]);
          pu.y = pack_bf16x2_hw(acc[i][1][4 * q + 2], acc[i][1][4 * q + 3]);
          uint16_t *gu = reinterpret_cast<uint16_t *>(a.out2) + orow * a.ldg + col;
          *reinterpret_cast<uint2 *>(gu) = pg;
          *reinterpret_cast<uint2 *>(gu + a.ncols) = pu;
        }
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float gs = acc[i][0][4 * q + e], us = acc[i][1][4 * q + e];
          if constexpr (FP8) {
            gs *= bsc[0][q][e];
            us *= bsc[1][q][e];
          }
          v[e] = glu_act_fast(gs, us, a.act, a.beta_g, a.beta_u);
        }
        uint2 pk;
        pk.x = pack_bf16x2_hw(v[0], v[1]);
        pk.y = pack_bf16x2_hw(v[2], v[3]);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + orow * a.ldo + col) = pk;
      }
    } else {
      // The epilogue's own inputs (G and U; the fp32 addends) for this row
      // block are all loaded before the first store, so their latencies
      // overlap instead of queueing behind each store.
      uint2 gpre[2][4], upre[2][4];
      float4 apre0[2][4], apre1[2][4];
      if constexpr (EPI == EP_GLU_BWD || EPI == EP_ADD_BF16) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t col = n_tile * BN + wn * 64 + j * 32 + 8 * q + 4 * khalf;
            if (col >= a.ncols) continue;
            if constexpr (EPI == EP_GLU_BWD) {
              gpre[j][q] = *reinterpret_cast<const uint2 *>(a.gsrc + orow * a.ldg + col);
              upre[j][q] = *reinterpret_cast<const uint2 *>(a.usrc + orow * a.ldg + col);
            } else {
              apre0[j][q] = *reinterpret_cast<const float4 *>(a.add0 + orow * a.ldo + col);
              if (a.add1 != nullptr)
                apre1[j][q] = *reinterpret_cast<const float4 *>(a.add1 + orow * a.ldo + col);
            }
          }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = n_tile * BN + wn * 64 + j * 32 + 8 * q + 4 * khalf;
          if (col >= a.ncols) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          if constexpr (EPI == EP_F32) {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + orow * a.ldo + col) =
                make_float4(v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EP_GLU_BWD) {
            // v = dH at (orow, col..col+3): the activation's backward with
            // the recomputed G and U of the same entries.
            const uint2 gr = gpre[j][q];
            const uint2 ur = upre[j][q];
            const float gv[4] = {__uint_as_float(gr.x << 16), __uint_as_float(gr.x & 0xFFFF0000u),
                                 __uint_as_float(gr.y << 16), __uint_as_float(gr.y & 0xFFFF0000u)};
            const float uv[4] = {__uint_as_float(ur.x << 16), __uint_as_float(ur.x & 0xFFFF0000u),
                                 __uint_as_float(ur.y << 16), __uint_as_float(ur.y & 0xFFFF0000u)};
            float dg[4], du[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              glu_act_backward_fast(gv[e], uv[e], v[e], a.act, a.beta_g, a.beta_u, dg[e],
                                    du[e]);
            uint2 pg, pu;
            pg.x = pack_bf16x2_hw(dg[0], dg[1]);
            pg.y = pack_bf16x2_hw(dg[2], dg[3]);
            pu.x = pack_bf16x2_hw(du[0], du[1]);
            pu.y = pack_bf16x2_hw(du[2], du[3]);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + orow * a.ldo + col) =
                pg;
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out2) + orow * a.ldo + col) =
                pu;
          } else {
            if constexpr (EPI == EP_ADD_BF16) {
              const float4 p0 = apre0[j][q];
              v[0] += p0.x; v[1] += p0.y; v[2] += p0.z; v[3] += p0.w;
              if (a.add1 != nullptr) {
                const float4 p1 = apre1[j][q];
                v[0] += p1.x; v[1] += p1.y; v[2] += p1.z; v[3] += p1.w;
              }
            }
            uint2 pk;
            pk.x = pack_bf16x2_hw(v[0], v[1]);
            pk.y = pack_bf16x2_hw(v[2], v[3]);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + orow * a.ldo + col) =
                pk;
          }
        }
      }
    }
  }
}

// tile_start[g] = sum_{g' < g} ceil(M_g' / bm), M_g = kept rows of group g.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t *__restrict__ kept_offsets,
                                                           int G, int bm,
                                                           int32_t *__restrict__ tile_start) {
  __shared__ int tmp[1024];
  int run = 0;  // carried across rounds of 1024 groups
  for (int base = 0; base < G; base += 1024) {
    const int g = base + threadIdx.x;
    const int m = (g < G) ? kept_offsets[g + 1] - kept_offsets[g] : 0;
    tmp[threadIdx.x] = (m + bm - 1) / bm;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int add = (int)threadIdx.x >= o ? tmp[threadIdx.x - o] : 0;
      __syncthreads();
      tmp[threadIdx.x] += add;
      __syncthreads();
    }
    if (g < G) tile_start[g + 1] = run + tmp[threadIdx.x];
    run += tmp[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) tile_start[0] = 0;
}

// One launch per (epilogue, tile height) pair, written out so that every
// kernel instance is referenced from a non-template function.
hipError_t launch_kernel(const GemmArgs &a, int epi, int bm, int64_t grid, hipStream_t st) {
  const dim3 g(grid), b(kThreads);
  if (a.kseg != nullptr || a.kchunk > 0) {
    if (epi != EP_F32 || bm != 256) return hipErrorInvalidValue;
    if (a.kseg == nullptr && (a.mode != GM_DENSE || a.kchunk % 128 != 0)) return hipErrorInvalidValue;
    grouped_gemm_kernel<EP_F32, 256, false, true><<<g, b, 0, st>>>(a);
    return hipGetLastError();
  }
  if (a.bt) {
    if (epi != EP_GLU_BWD && epi != EP_F32) return hipErrorInvalidValue;
    if (a.ncols % 8 != 0 || a.ldbt % 8 != 0 || a.ksplit % BK != 0) return hipErrorInvalidValue;
    if (epi == EP_GLU_BWD) {
      if (bm == 192) grouped_gemm_kernel<EP_GLU_BWD, 192, false, false, true><<<g, b, 0, st>>>(a);
      else grouped_gemm_kernel<EP_GLU_BWD, 256, false, false, true><<<g, b, 0, st>>>(a);
    } else {
      if (bm == 192) grouped_gemm_kernel<EP_F32, 192, false, false, true><<<g, b, 0, st>>>(a);
      else grouped_gemm_kernel<EP_F32, 256, false, false, true><<<g, b, 0, st>>>(a);
    }
    return hipGetLastError();
  }
  if (epi == EP_GLU_SAVE) {
    if (a.bscale != nullptr) return hipErrorInvalidValue;
    if (bm == 192) grouped_gemm_kernel<EP_GLU_SAVE, 192><<<g, b, 0, st>>>(a);
    else grouped_gemm_kernel<EP_GLU_SAVE, 256><<<g, b, 0, st>>>(a);
    return hipGetLastError();
  }
  if (epi == EP_GU || epi == EP_GLU_BWD) {
    if (epi == EP_GU) {
      if (bm == 192) grouped_gemm_kernel<EP_GU, 192><<<g, b, 0, st>>>(a);
      else grouped_gemm_kernel<EP_GU, 256><<<g, b, 0, st>>>(a);
    } else {
      if (bm == 192) grouped_gemm_kernel<EP_GLU_BWD, 192><<<g, b, 0, st>>>(a);
      else grouped_gemm_kernel<EP_GLU_BWD, 256><<<g, b, 0, st>>>(a);
    }
    return hipGetLastError();
  }
  if (a.mx4) {
    if ((epi != EP_GLU && epi != EP_F32) || a.bscale == nullptr || a.K % 128 != 0)
      return hipErrorInvalidValue;
    if (epi == EP_GLU) {
      if (bm == 192) grouped_gemm_kernel<EP_GLU, 192, false, false, false, true><<<g, b, 0, st>>>(a);
      else grouped_gemm_kernel<EP_GLU, 256, false, false, false, true><<<g, b, 0, st>>>(a);
    } else {
      if (bm == 192) grouped_gemm_kernel<EP_F32, 192, false, false, false, true><<<g, b, 0, st>>>(a);
      else grouped_gemm_kernel<EP_F32, 256, false, false, false, true><<<g, b, 0, st>>>(a);
    }
    return hipGetLastError();
  }
  if (a.bscale != nullptr) {
    if (epi != EP_GLU && epi != EP_F32) return hipErrorInvalidValue;
    if (epi == EP_GLU) {
      if (bm == 192) grouped_gemm_kernel<EP_GLU, 192, true><<<g, b, 0, st>>>(a);
      else grouped_gemm_kernel<EP_GLU, 256, true><<<g, b, 0, st>>>(a);
    } else {
      if (bm == 192) grouped_gemm_kernel<EP_F32, 192, true><<<g, b, 0, st>>>(a);
      else grouped_gemm_kernel<EP_F32, 256, true><<<g, b, 0, st>>>(a);
    }
    return hipGetLastError();
  }
  if (bm == 192) {
    switch (epi) {
      case EP_GLU: grouped_gemm_kernel<EP_GLU, 192><<<g, b, 0, st>>>(a); break;
      case EP_F32: grouped_gemm_kernel<EP_F32, 192><<<g, b, 0, st>>>(a); break;
      case EP_BF16: grouped_gemm_kernel<EP_BF16, 192><<<g, b, 0, st>>>(a); break;
      default: grouped_gemm_kernel<EP_ADD_BF16, 192><<<g, b, 0, st>>>(a); break;
    }
  } else {
    switch (epi) {
      case EP_GLU: grouped_gemm_kernel<EP_GLU, 256><<<g, b, 0, st>>>(a); break;
      case EP_F32: grouped_gemm_kernel<EP_F32, 256><<<g, b, 0, st>>>(a); break;
      case EP_BF16: grouped_gemm_kernel<EP_BF16, 256><<<g, b, 0, st>>>(a); break;
      default: grouped_gemm_kernel<EP_ADD_BF16, 256><<<g, b, 0, st>>>(a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

int gemm_pick_bm(double rows_per_group) {
  // The m-tile height that pads an average group least (256 on ties).
  if (rows_per_group <= 0) return 256;
  const double w256 = std::ceil(rows_per_group / 256.0) * 256.0 - rows_per_group;
  const double w192 = std::ceil(rows_per_group / 192.0) * 192.0 - rows_per_group;
  return w192 < w256 ? 192 : 256;
}

int64_t gemm_mtile_bound(int64_t rows_total, int groups, int bm) {
  return (rows_total + bm - 1) / bm + groups;
}

hipError_t launch_tile_prefix(const int32_t *kept_offsets, int G, int bm, int32_t *tile_start,
                              hipStream_t st) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, kept_offsets, G, bm,
                     tile_start);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, int epi, int64_t mtiles_bound, hipStream_t st) {
  const int bm = a.bm == 192 ? 192 : 256;
  const int64_t NT = (epi == EP_GLU || epi == EP_GU || epi == EP_GLU_SAVE)
                         ? (a.ncols + 127) / 128
                                                      : (a.ncols + BN - 1) / BN;
  int64_t tiles;
  if (a.mode == GM_DENSE) tiles = (int64_t)a.G * ((a.M_dense + bm - 1) / bm) * NT;
  else tiles = mtiles_bound * NT;
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  return launch_kernel(a, epi, bm, grid, st);
}

}  // namespace moe
