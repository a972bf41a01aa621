// gemm_tiled.hip -- projections with many rows per weight matrix (prefill).
//
// C[rows][n] = sum_k A[row][k] * B[n][k] on bf16 MFMA 16x16x32 with fp32
// accumulation, for the expert gate/up (+ SwiGLU) and down projections
// (steps A5, A6; MXFP4 weights) and the pooler/unpooler (A4, A8; bf16).
//
// Workgroup tile: 64 rows x (4 x 64) weight rows (x (4 x 32) for bf16
// weights), four wavefronts. The A rows (gathered latent rows, h rows or
// input rows, bf16) are copied straight from global memory into a
// double-buffered LDS tile shared by the four wavefronts (buffer loads with
// the LDS destination, so no registers hold them in flight); the tile is
// XOR-swizzled so that the 16 rows one ds_read_b128 touches fall in distinct
// banks. Every wavefront owns its weight rows for all 64 tile rows and reads
// them into registers one stage ahead, where MXFP4 is decoded (gfx950 scaled
// FP4 -> bf16 conversion) once per element.
//
// Expert work comes from the row-tile list of the grouping step (expert,
// first sorted row; 64 rows at most). A tile runs the MFMAs of its first
// 4, 2 or 1 fragments of 16 rows (the smallest count covering its rows);
// the choice is made once per tile, so the inner loop has no branches.
// Workgroup ids are remapped so that the column tiles of one row tile run
// on one XCD (ids congruent mod 8) and share its activation rows in that
// L2, row tiles dealt to the XCDs in turn (the grid is sized for the most
// tiles the grouping can make; the tiles that exist spread over all XCDs).
//
// Reduction order inside a 128-element chunk, as in the decode kernels: lane
// group g = lane/16 owns elements [32g, 32g+32); MFMA j takes 32g+8j .. +7.
// The pipeline moves two chunks (256 elements) per stage; K must be a
// multiple of 256.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBM = 64;         // rows of a dense tile
constexpr int kWaves = 4;
constexpr int kStageK = 256;    // reduction elements per pipeline stage (two chunks)

// Weight rows per wavefront: 64 for MXFP4 (16 code bytes per row and chunk),
// 32 for bf16 (64 bytes per row and chunk), to fit 2 workgroups per CU.
template <int BFMT>
constexpr int wave_cols() { return is_fp4(BFMT) ? 64 : 32; }

template <int BFMT, int EPI>
__global__ __launch_bounds__(64 * kWaves, 2) void tiled_kernel(TiledArgs p) {
  constexpr int kRows = (EPI == EPI_BF16) ? kBM : kTileRows;  // tile rows
  constexpr int kMF = kRows / 16;                               // 16-row A fragments
  constexpr int kAP = kRows * 32 / (64 * kWaves);  // 1-KiB LDS blocks per wavefront and stage
  constexpr int kWN = wave_cols<BFMT>();
  constexpr int kNF = kWN / 16;  // 16-row weight fragments per wavefront
  __shared__ __attribute__((aligned(1024))) uint16_t As[2][kRows * 256];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;

  // ---- XCD-aware tile order: a row tile's column tiles on one XCD ----
  const int logical = xcd_tile(p.n_col_tiles);
  const int mt = logical / p.n_col_tiles, nt = logical % p.n_col_tiles;

  int row_begin, row_end, expert = 0;
  if (p.grouped) {
    if (mt >= p.counters[1]) return;
    expert = p.tiles[2 * mt];
    row_begin = p.tiles[2 * mt + 1];
    // (a tile list no grouping of this call has written is skipped)
    if (expert < 0 || expert >= p.n_experts || row_begin < 0 || row_begin >= p.n_routes) return;
    row_end = min(row_begin + kTileRows, min(p.offsets[expert + 1], p.n_routes));
    if (row_end <= row_begin) return;
    // (the split into light and heavy experts: a light one is the streaming kernel's)
    if (p.offsets[expert + 1] - p.offsets[expert] <= p.min_rows) return;
  } else {
    if (mt * kBM >= p.m_total) return;
    row_begin = mt * kBM;
    row_end = min(p.m_total, row_begin + kBM);
  }
  const int nrows = row_end - row_begin;  // >= 1
  const uint32_t K = static_cast<uint32_t>(p.K);

  // ---- A: the stage's tile (kBM rows x 256 elements, 512 bytes per row) is
  // copied straight into LDS, 16-byte piece c of row r stored at position
  // r*32 + (c ^ (r % 16)): the 16 rows one ds_read_b128 touches then start in
  // distinct banks. Wavefront w copies LDS blocks w*kAP .. w*kAP+kAP-1 (64
  // pieces each); a_off[i] is this lane's source offset for block i.
  const rsrc_t a_r = make_rsrc(p.a, p.a_bytes);
  uint32_t a_off[kAP];
#pragma unroll
  for (int i = 0; i < kAP; ++i) {
    const int piece = (wave * kAP + i) * 64 + lane;
    const int r = piece >> 5, c = (piece & 31) ^ (r & 15);
    const int pos = row_begin + r;
    a_off[i] = kOutOfRange;
    if (pos < row_end) {
      const int ar = p.a_gather ? p.sorted[pos] / p.topk : pos;
      a_off[i] = static_cast<uint32_t>(ar) * K * 2 + c * 16;
    }
  }
  const uint32_t lds_a0 = static_cast<uint32_t>(reinterpret_cast<size_t>(
      (__attribute__((address_space(3))) uint16_t*)(&As[0][0])));

  // ---- B: one descriptor per expert (or the dense matrix) ----
  constexpr int SB = scale_block(BFMT);  // elements per scale byte
  rsrc_t bq_r, bs_r;
  if (is_fp4(BFMT)) {
    const size_t rows = static_cast<size_t>(p.b_rows_per_expert);
    bq_r = make_rsrc(p.b_codes + expert * rows * (K / 2), static_cast<uint32_t>(rows * (K / 2)));
    bs_r = make_rsrc(p.b_scales + expert * rows * (K / SB), static_cast<uint32_t>(rows * (K / SB)));
  } else {
    bq_r = make_rsrc(p.b_bf16, p.b_bytes);
    bs_r = bq_r;
  }
  uint32_t bq_off[kNF], bs_off[kNF];
  int col_base;  // first output column of this wavefront
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    int r;
    if (EPI == EPI_SWIGLU) {
      // fragments 0 .. kNF/2-1: gate rows; kNF/2 .. kNF-1: the matching up rows
      col_base = nt * (kWaves * kWN / 2) + wave * (kWN / 2);
      r = (f / (kNF / 2)) * p.inter + col_base + (f % (kNF / 2)) * 16 + nl;
    } else {
      col_base = nt * (kWaves * kWN) + wave * kWN;
      r = col_base + f * 16 + nl;
    }
    if (is_fp4(BFMT)) {
      bq_off[f] = r * (K / 2) + g * 16;
      bs_off[f] = r * (K / SB) + (BFMT == B_NVFP4 ? 4 * (g >> 1) : 0);
    } else {
      bq_off[f] = r * K * 2 + g * 64;
      bs_off[f] = 0;
    }
  }

  f32x4 acc[kMF][kNF];
#pragma unroll
  for (int m = 0; m < kMF; ++m)
#pragma unroll
    for (int f = 0; f < kNF; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int BQ = is_fp4(BFMT) ? 1 : 4;  // 16-byte loads per row and chunk
  uint4 bq[2][2][kNF][BQ];  // [buffer][chunk of the stage][fragment]
  // per chunk: its 4 E8M0 bytes, or the dword of its 8 E4M3 bytes that holds
  // the lane group's two (bytes 2g, 2g+1 in dword g/2)
  uint32_t bs[2][2][kNF];
  auto load_a = [&](auto stage_tag, int st) __attribute__((always_inline)) {
    constexpr int stage = decltype(stage_tag)::value;
#pragma unroll
    for (int i = 0; i < kAP; ++i) {
      const uint32_t lds = __builtin_amdgcn_readfirstlane(
          lds_a0 + stage * (kRows * 512) + (wave * kAP + i) * 1024);
      lds_copy16(a_r, a_off[i] + st * 512, lds);
    }
  };
  auto load_b = [&](auto buf_tag, int st) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_tag)::value;
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      if (is_fp4(BFMT)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) bq[buf][h][f][0] = buf_load16<kAuxDefault>(bq_r, bq_off[f] + st * 128 + h * 64);
        if (BFMT == B_NVFP4) {  // 8 scale bytes per chunk: the lane's dword of each
          bs[buf][0][f] = buf_load4<kAuxDefault>(bs_r, bs_off[f] + st * 16);
          bs[buf][1][f] = buf_load4<kAuxDefault>(bs_r, bs_off[f] + st * 16 + 8);
        } else {
          const uint2 sv = buf_load8b<kAuxDefault>(bs_r, bs_off[f] + st * 8);  // scales of both chunks
          bs[buf][0][f] = sv.x;
          bs[buf][1][f] = sv.y;
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) bq[buf][h][f][j] = buf_load16<kAuxDefault>(bq_r, bq_off[f] + st * 512 + h * 256 + j * 16);
        bs[buf][0][f] = bs[buf][1][f] = 0;
      }
    }
  };
  // MFMAs of one stage for the first LIVE 16-row fragments, branch-free:
  // per 32-element sub-step, the LIVE A fragments from LDS, the kNF decoded
  // weight fragments, then LIVE x kNF independent MFMAs.
  auto compute = [&](auto stage_tag, auto live_tag) __attribute__((always_inline)) {
    constexpr int stage = decltype(stage_tag)::value;  // LDS stage = B buffer
    constexpr int buf = stage;
    constexpr int LIVE = decltype(live_tag)::value;
    const uint16_t* as = As[stage];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 bv[kNF];
#pragma unroll
        for (int f = 0; f < kNF; ++f) {
          if (is_fp4(BFMT)) {
            // MXFP4: byte g of the chunk's scales; NVFP4: byte 2g + j/2 of
            // its 8 (the E4M3 value; the tensor's scale multiplies the sums)
            float sc;
            if constexpr (BFMT == B_NVFP4)
              sc = e4m3_to_f32((bs[buf][h][f] >> (16 * (g & 1) + 8 * (j >> 1))) & 0xFFu);
            else
              sc = e8m0_to_f32((bs[buf][h][f] >> (8 * g)) & 0xFFu);
            const uint4 q = bq[buf][h][f][0];
            const uint32_t d = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
            bv[f] = BFMT == B_NVFP4 ? nvfp4x8_to_bf16(d, sc) : mxfp4x8_to_bf16(d, sc);
          } else {
            bv[f] = as_bf16x8(bq[buf][h][f][j]);
          }
        }
        // piece h*16 + g*4 + j of rows m*16 + nl (swizzled by nl)
        const uint16_t* arow = &as[nl * 256 + ((h * 16 + g * 4 + j) ^ nl) * 8];
        bf16x8 av[LIVE];
#pragma unroll
        for (int m = 0; m < LIVE; ++m) av[m] = as_bf16x8(*reinterpret_cast<const uint4*>(arow + m * 16 * 256));
#pragma unroll
        for (int m = 0; m < LIVE; ++m)
#pragma unroll
          for (int f = 0; f < kNF; ++f) acc[m][f] = mfma16x16x32(av[m], bv[f], acc[m][f]);
      }
    }
  };

  // Stages of 256 reduction elements, two per iteration so that the buffers
  // have fixed names: issue stage s+1's copies (A into the other LDS tile, B
  // into the other register buffer), compute stage s, wait for the copies,
  // barrier. Copies past the last stage repeat the last stage (unused), so
  // the loop has no conditional loads.
  const int nst = p.K / kStageK;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto kloop = [&](auto live_tag) __attribute__((always_inline)) {
    load_a(I0{}, 0);
    load_b(I0{}, 0);
    wait_vm_keep<0>();
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
      load_a(I1{}, min(st + 1, nst - 1));
      load_b(I1{}, min(st + 1, nst - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(I0{}, live_tag);
      wait_vm_keep<0>();
      __syncthreads();
      if (st + 1 >= nst) break;
      load_a(I0{}, min(st + 2, nst - 1));
      load_b(I0{}, min(st + 2, nst - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(I1{}, live_tag);
      wait_vm_keep<0>();
      __syncthreads();
    }
  };
  const int mf_live = (nrows + 15) / 16;
  if (kMF > 4 && mf_live > 4)
    kloop(std::integral_constant<int, kMF>{});
  else if (mf_live > 2)
    kloop(std::integral_constant<int, 4>{});
  else if (mf_live > 1)
    kloop(std::integral_constant<int, 2>{});
  else
    kloop(std::integral_constant<int, 1>{});

  // ---- epilogue ----
  // NVFP4: the tensor's global scale, applied to the fp32 sums
  const float gs = (BFMT == B_NVFP4) ? p.b_global[expert] : 1.0f;
#pragma unroll
  for (int m = 0; m < kMF; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = row_begin + m * 16 + 4 * g + i;
      if (pos >= row_end) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int f = 0; f < kNF / 2; ++f) {
          const float gt = acc[m][f][i] * gs, up = acc[m][f + kNF / 2][i] * gs;
          const float silu = gt / (1.0f + expf(-gt));
          static_cast<uint16_t*>(p.out)[static_cast<size_t>(pos) * p.ldo + col_base + f * 16 + nl] =
              f32_to_bf16(silu * up);
        }
      } else if (EPI == EPI_F32_SCATTER) {
        float* dst = static_cast<float*>(p.out) + static_cast<size_t>(p.sorted[pos]) * p.ldo + col_base + nl;
#pragma unroll
        for (int f = 0; f < kNF; ++f) dst[f * 16] = acc[m][f][i] * gs;
      } else {
        uint16_t* dst = static_cast<uint16_t*>(p.out) + static_cast<size_t>(pos) * p.ldo + col_base + nl;
#pragma unroll
        for (int f = 0; f < kNF; ++f) dst[f * 16] = f32_to_bf16(acc[m][f][i]);
      }
    }
  }
}

template <int BFMT, int EPI>
hipError_t launch_tiled(const TiledArgs& a, int n_row_tiles, hipStream_t st) {
  static_assert(kWaves * wave_cols<BFMT>() >= 64, "tile width");
  const int n = n_row_tiles * a.n_col_tiles;
  const dim3 grid(xcd_grid(n, a.n_col_tiles)), block(64 * kWaves);
  MOE_LAUNCH((tiled_kernel<BFMT, EPI>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_tiled(const uint16_t* a, const uint16_t* b, uint16_t* out, int M, int N,
                              int K, hipStream_t st, float* part) {
  // the LDS-staged kernel when its tiles (with a K split and the partial
  // sums in `part` when too few) fill the GPU
  const int S = dense_splits(M, N, K);
  if (S == 1 || (S > 1 && part)) return launch_dense_lds(a, b, out, M, N, K, st, part);
  TiledArgs p{};
  p.a = a;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(M) * K * 2);
  p.m_total = M;
  p.b_bf16 = b;
  p.b_bytes = static_cast<uint32_t>(static_cast<size_t>(N) * K * 2);
  p.K = K;
  p.out = out;
  p.ldo = N;
  p.n_col_tiles = N / (kWaves * wave_cols<B_BF16>());
  return launch_tiled<B_BF16, EPI_BF16>(p, (M + kBM - 1) / kBM, st);
}

hipError_t launch_gateup_tiled(const ExpertGemm& x, hipStream_t st) {
  TiledArgs p{};
  p.grouped = 1;
  p.a = x.lat;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(x.tokens) * x.latent * 2);
  p.a_gather = 1;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.offsets = x.offsets;
  p.counters = x.counters;
  p.tiles = x.tiles;
  p.b_codes = x.w13_codes;
  p.b_scales = x.w13_scales;
  p.b_rows_per_expert = 2 * x.inter;
  p.K = x.latent;
  p.inter = x.inter;
  p.out = x.h;
  p.ldo = x.inter;
  p.n_col_tiles = x.inter / (kWaves * wave_cols<B_MXFP4>() / 2);
  p.b_global = x.w13_global;
  p.n_experts = x.n_experts;
  p.n_routes = x.tokens * x.topk;
  p.min_rows = x.split_rows;
  return x.nvfp4 ? launch_tiled<B_NVFP4, EPI_SWIGLU>(p, x.max_tiles, st)
                 : launch_tiled<B_MXFP4, EPI_SWIGLU>(p, x.max_tiles, st);
}

hipError_t launch_down_tiled(const ExpertGemm& x, hipStream_t st) {
  TiledArgs p{};
  p.grouped = 1;
  p.a = x.h;
  p.a_bytes = static_cast<uint32_t>(static_cast<size_t>(x.tokens) * x.topk * x.inter * 2);
  p.a_gather = 0;
  p.sorted = x.sorted;
  p.topk = x.topk;
  p.offsets = x.offsets;
  p.counters = x.counters;
  p.tiles = x.tiles;
  p.b_codes = x.w2_codes;
  p.b_scales = x.w2_scales;
  p.b_rows_per_expert = x.latent;
  p.K = x.inter;
  p.out = x.rows;
  p.ldo = x.latent;
  p.n_col_tiles = x.latent / (kWaves * wave_cols<B_MXFP4>());
  p.b_global = x.w2_global;
  p.n_experts = x.n_experts;
  p.n_routes = x.tokens * x.topk;
  p.min_rows = x.split_rows;
  return x.nvfp4 ? launch_tiled<B_NVFP4, EPI_F32_SCATTER>(p, x.max_tiles, st)
                 : launch_tiled<B_MXFP4, EPI_F32_SCATTER>(p, x.max_tiles, st);
}

}  // namespace moe
