// CPU bounds check of the HIP kernel sources (test infrastructure).
//
// The kernel headers are compiled as host C++ (see shim/hip/hip_runtime.h)
// and every thread of every workgroup of a launch is run one after another
// on buffers that sit flush against inaccessible guard regions of 8 GiB on
// each side.  Any read or write outside a buffer -- including a 32-bit
// offset that wrapped below zero -- lands in a guard region and raises
// SIGSEGV; the caller treats a non-zero exit as a failure.  Results are not
// checked here (barriers are no-ops), only addresses.
//
// usage: emul <variant> <nx> <ny> <nz> <wide:0|1> <grid:0=as launched> <end_aligned:0|1> <planes>
//   variant: fused | fused_nostream | fused_h | fused_nostream_h | pair | pair_nostream |
//            pair_h | pair_nostream_h | reg_march | point | two_kernel | lds_march |
//            lds_march_32x4 | lds_march_32x8 | lds_march_32x16 | lds_march_64x8 |
//            primal | primal_h | gap | gap_pair | tb2 | tb2_h | cube | cube_32x8x2 | cube_64x8x1 |
//            cube_8x8x8 | cube_32x4x4
//   (the pair variants need an even nx; with an odd one they report "ok" without running)
//   wide: 1 instantiates the 64-bit offset / index path regardless of size
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/mman.h>

#include <type_traits>

#include "tv_fgp_ablation_kernels.hpp"
#include "tv_fgp_device.hpp"
#include "tv_fgp_fused_kernel.hpp"
#include "tv_fgp_gap_kernel.hpp"
#include "tv_fgp_lds_kernel.hpp"
#include "tv_fgp_pair_kernel.hpp"
#include "tv_fgp_tb2_kernel.hpp"
#include "tv_fgp_tb3_kernel.hpp"
#include "tv_fgp_cube_kernel.hpp"

thread_local EmulDim3 threadIdx, blockIdx, gridDim, blockDim;

namespace {

const size_t kGuard = size_t(8) << 30;

float *guarded(size_t bytes, bool end_aligned, unsigned seed) {
  const size_t page = 4096;
  const size_t span = (bytes + page - 1) / page * page;
  void *r = mmap(nullptr, kGuard + span + kGuard, PROT_NONE,
                 MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
  if (r == MAP_FAILED) {
    perror("mmap");
    exit(3);
  }
  char *mid = (char *)r + kGuard;
  if (mprotect(mid, span, PROT_READ | PROT_WRITE) != 0) {
    perror("mprotect");
    exit(3);
  }
  // A buffer of binary16 volumes may be only 2-byte aligned at its start, so
  // the fill goes byte by byte (small floats, or binary16 halves of them).
  char *p = end_aligned ? mid + span - bytes : mid;
  unsigned s = seed * 2654435761u + 1u;
  for (size_t i = 0; i < bytes; i += sizeof(float)) {
    s = s * 1664525u + 1013904223u;
    const float v = ((float)(s >> 8) / 16777216.0f - 0.5f) * 0.1f;
    memcpy(p + i, &v, bytes - i < sizeof(float) ? bytes - i : sizeof(float));
  }
  return (float *)p;
}

template <typename F>
void run_grid(unsigned grid, unsigned block, F &&thread_body) {
  gridDim = {grid, 1, 1};
  blockDim = {block, 1, 1};
  for (unsigned bl = 0; bl < grid; ++bl) {
    for (unsigned th = 0; th < block; ++th) {
      blockIdx = {bl, 0, 0};
      threadIdx = {th, 0, 0};
      thread_body();
    }
  }
}

unsigned pick_grid(int64_t ntiles, unsigned override_grid) {
  if (override_grid) return override_grid;
  return tvfgp::grid_for(ntiles);
}

struct Bufs {
  float *b, *p[3], *ri[3], *ro[3], *z, *po[3];
};

template <typename I, int TX, int TY>
void run_march(const Bufs &v, int64_t nx, int64_t ny, int64_t nz, unsigned grid, int64_t planes) {
  const tvfgp::Geometry<I> g = tvfgp::march_geometry<I>(nx, ny, nz, planes, TX, TY);
  run_grid(pick_grid(g.ntiles, grid), TX * TY, [&] {
    tvfgp::lds_march_kernel<I, TX, TY>(v.b, v.p[0], v.p[1], v.p[2], v.ri[0], v.ri[1], v.ri[2],
                                       v.ro[0], v.ro[1], v.ro[2], 0.01f, 8.3f, 0.5f, g);
  });
}

template <typename I, typename Off, typename S>
void run_tb3(const Bufs &v, int64_t nx, int64_t ny, int64_t nz, unsigned grid, int64_t planes) {
  const auto g = tvfgp::tb_geometry<I, Off>(nx, ny, nz, planes);
  S *p[3], *po[3], *ri[3], *ro[3];
  for (int a = 0; a < 3; ++a) {
    p[a] = (S *)v.p[a];
    po[a] = (S *)v.po[a];
    ri[a] = (S *)v.ri[a];
    ro[a] = (S *)v.ro[a];
  }
  run_grid(pick_grid(g.ntiles, grid), tvfgp::kTbBlock, [&] {
    tvfgp::tb3_kernel<I, Off, S>(v.b, p[0], p[1], p[2], po[0], po[1], po[2], ri[0], ri[1], ri[2],
                                 ro[0], ro[1], ro[2], 0.01f, 8.3f, 0.3f, 0.5f, 0.6f, g);
  });
}

template <typename I, typename Off, typename S>
void run_tb2(const Bufs &v, int64_t nx, int64_t ny, int64_t nz, unsigned grid, int64_t planes) {
  const auto g = tvfgp::tb_geometry<I, Off>(nx, ny, nz, planes);
  S *p[3], *po[3], *ri[3], *ro[3];
  for (int a = 0; a < 3; ++a) {
    p[a] = (S *)v.p[a];
    po[a] = (S *)v.po[a];
    ri[a] = (S *)v.ri[a];
    ro[a] = (S *)v.ro[a];
  }
  run_grid(pick_grid(g.ntiles, grid), tvfgp::kTbBlock, [&] {
    tvfgp::tb2_kernel<I, Off, S>(v.b, p[0], p[1], p[2], po[0], po[1], po[2], ri[0], ri[1], ri[2],
                                 ro[0], ro[1], ro[2], 0.01f, 8.3f, 0.3f, 0.5f, g);
  });
}

template <typename I, typename Off, typename S>
void run_pair(const Bufs &v, int64_t nx, int64_t ny, int64_t nz, unsigned grid,
              bool stream_p) {
  const auto g = tvfgp::pair_geometry<I, Off>(nx, ny, nz);
  const unsigned gr = pick_grid(g.ntiles, grid);
  S *p[3], *ri[3], *ro[3];
  for (int a = 0; a < 3; ++a) {
    p[a] = (S *)v.p[a];
    ri[a] = (S *)v.ri[a];
    ro[a] = (S *)v.ro[a];
  }
  if (stream_p)
    run_grid(gr, tvfgp::kPairBlock, [&] {
      tvfgp::fused_pair_kernel<I, Off, true, S>(v.b, p[0], p[1], p[2], ri[0], ri[1], ri[2],
                                                ro[0], ro[1], ro[2], 0.01f, 8.3f, 0.5f, g);
    });
  else
    run_grid(gr, tvfgp::kPairBlock, [&] {
      tvfgp::fused_pair_kernel<I, Off, false, S>(v.b, p[0], p[1], p[2], ri[0], ri[1], ri[2],
                                                 ro[0], ro[1], ro[2], 0.01f, 8.3f, 0.5f, g);
    });
}

template <typename I, typename Off, typename S>
void run_fused(const Bufs &v, int64_t nx, int64_t ny, int64_t nz, unsigned grid,
               bool stream_p) {
  const auto g = tvfgp::zx_geometry<I, Off>(nx, ny, nz);
  const unsigned gr = pick_grid(g.ntiles, grid);
  S *p[3], *ri[3], *ro[3];
  for (int a = 0; a < 3; ++a) {
    p[a] = (S *)v.p[a];
    ri[a] = (S *)v.ri[a];
    ro[a] = (S *)v.ro[a];
  }
  if (stream_p)
    run_grid(gr, tvfgp::kZxBlock, [&] {
      tvfgp::fused_zx_kernel<I, Off, true, S>(v.b, p[0], p[1], p[2], ri[0], ri[1], ri[2],
                                              ro[0], ro[1], ro[2], 0.01f, 8.3f, 0.5f, g);
    });
  else
    run_grid(gr, tvfgp::kZxBlock, [&] {
      tvfgp::fused_zx_kernel<I, Off, false, S>(v.b, p[0], p[1], p[2], ri[0], ri[1], ri[2],
                                               ro[0], ro[1], ro[2], 0.01f, 8.3f, 0.5f, g);
    });
}

template <typename I, int TX, int TY, int TZ>
void run_cube(const Bufs &v, int64_t nx, int64_t ny, int64_t nz, unsigned grid) {
  const auto g = tvfgp::cube_geometry<I, TX, TY, TZ>(nx, ny, nz);
  run_grid(pick_grid(g.ntiles, grid), tvfgp::kCubeBlock, [&] {
    tvfgp::cube_kernel<I, TX, TY, TZ>(v.b, v.p[0], v.p[1], v.p[2], v.ri[0], v.ri[1], v.ri[2],
                                      v.ro[0], v.ro[1], v.ro[2], 0.01f, 8.3f, 0.5f, g);
  });
}

template <typename I>
void run_ablation(const char *variant, const Bufs &v, int64_t nx, int64_t ny, int64_t nz,
                  unsigned grid, int64_t planes) {
  using namespace tvfgp;
  if (!strcmp(variant, "cube")) {
    run_cube<I, 16, 8, 4>(v, nx, ny, nz, grid);
  } else if (!strcmp(variant, "cube_32x8x2")) {
    run_cube<I, 32, 8, 2>(v, nx, ny, nz, grid);
  } else if (!strcmp(variant, "cube_64x8x1")) {
    run_cube<I, 64, 8, 1>(v, nx, ny, nz, grid);
  } else if (!strcmp(variant, "cube_8x8x8")) {
    run_cube<I, 8, 8, 8>(v, nx, ny, nz, grid);
  } else if (!strcmp(variant, "cube_32x4x4")) {
    run_cube<I, 32, 4, 4>(v, nx, ny, nz, grid);
  } else if (!strcmp(variant, "reg_march")) {
    const Geometry<I> g = make_geometry<I>(nx, ny, nz, planes);
    run_grid(pick_grid(g.ntiles, grid), kBlock, [&] {
      fused_march_kernel<I>(v.b, v.p[0], v.p[1], v.p[2], v.ri[0], v.ri[1], v.ri[2],
                            v.ro[0], v.ro[1], v.ro[2], 0.01f, 8.3f, 0.5f, g);
    });
  } else if (!strcmp(variant, "point")) {
    const Geometry<I> g = make_geometry<I>(nx, ny, nz, 1);
    run_grid(pick_grid(g.ntiles, grid), kBlock, [&] {
      fused_point_kernel<I>(v.b, v.p[0], v.p[1], v.p[2], v.ri[0], v.ri[1], v.ri[2],
                            v.ro[0], v.ro[1], v.ro[2], 0.01f, 8.3f, 0.5f, g);
    });
  } else if (!strcmp(variant, "primal_h")) {
    const Geometry<I> g = make_geometry<I>(nx, ny, nz, planes);
    run_grid(pick_grid(g.ntiles, grid), kBlock, [&] {
      primal_kernel<I, _Float16>(v.b, (const _Float16 *)v.ri[0], (const _Float16 *)v.ri[1],
                                 (const _Float16 *)v.ri[2], v.z, 0.01f, g);
    });
  } else if (!strcmp(variant, "two_kernel") || !strcmp(variant, "primal")) {
    const Geometry<I> g = make_geometry<I>(nx, ny, nz, planes);
    run_grid(pick_grid(g.ntiles, grid), kBlock, [&] {
      primal_kernel<I>(v.b, v.ri[0], v.ri[1], v.ri[2], v.z, 0.01f, g);
    });
    if (!strcmp(variant, "two_kernel"))
      run_grid(pick_grid(g.ntiles, grid), kBlock, [&] {
        dual_kernel<I>(v.z, v.p[0], v.p[1], v.p[2], v.ri[0], v.ri[1], v.ri[2], v.ro[0],
                       v.ro[1], v.ro[2], 8.3f, 0.5f, g);
      });
  } else if (!strcmp(variant, "gap")) {
    typedef typename std::conditional<sizeof(I) == 4, uint32_t, uint64_t>::type Off;
    const ZxGeometry<I, Off> g = zx_geometry<I, Off>(nx, ny, nz);
    const int count = grid ? (int)grid : gap_grid(nx, ny, nz);
    double *partial = (double *)guarded((size_t)count * 3 * sizeof(double), true, 99);
    double *out = (double *)guarded(3 * sizeof(double), true, 98);
    run_grid((unsigned)count, kZxBlock, [&] {
      gap_partial_kernel<I, Off>(v.b, v.p[0], v.p[1], v.p[2], 0.01f, g, partial);
    });
    run_grid(1, kGapFinalBlock, [&] { gap_final_kernel(partial, count, 0.01, out); });
  } else if (!strcmp(variant, "gap_pair")) {
    if (nx % 2 != 0) return;  // the pair kernel takes even nx only
    typedef typename std::conditional<sizeof(I) == 4, uint32_t, uint64_t>::type Off;
    const ZxGeometry<I, Off> g = gap_pair_geometry<I, Off>(nx, ny, nz);
    const int count = grid ? (int)grid : gap_pair_grid(nx, ny, nz);
    double *partial = (double *)guarded((size_t)count * 3 * sizeof(double), true, 99);
    double *out = (double *)guarded(3 * sizeof(double), true, 98);
    run_grid((unsigned)count, kPairBlock, [&] {
      gap_partial_pair_kernel<I, Off>(v.b, v.p[0], v.p[1], v.p[2], 0.01f, g, partial);
    });
    run_grid(1, kGapFinalBlock, [&] { gap_final_kernel(partial, count, 0.01, out); });
  } else if (!strcmp(variant, "lds_march")) {
    run_march<I, kTileX, kTileY>(v, nx, ny, nz, grid, planes);
  } else if (!strcmp(variant, "lds_march_32x4")) {
    run_march<I, 32, 4>(v, nx, ny, nz, grid, planes);
  } else if (!strcmp(variant, "lds_march_32x8")) {
    run_march<I, 32, 8>(v, nx, ny, nz, grid, planes);
  } else if (!strcmp(variant, "lds_march_32x16")) {
    run_march<I, 32, 16>(v, nx, ny, nz, grid, planes);
  } else if (!strcmp(variant, "lds_march_64x8")) {
    run_march<I, 64, 8>(v, nx, ny, nz, grid, planes);
  } else {
    fprintf(stderr, "unknown variant %s\n", variant);
    exit(2);
  }
}

}  // namespace

int main(int argc, char **argv) {
  if (argc != 9) {
    fprintf(stderr, "usage: emul variant nx ny nz wide grid end_aligned planes\n");
    return 2;
  }
  const char *variant = argv[1];
  const int64_t nx = atoll(argv[2]), ny = atoll(argv[3]), nz = atoll(argv[4]);
  const bool wide = atoi(argv[5]) != 0;
  const unsigned grid = (unsigned)atoi(argv[6]);
  const bool end_aligned = atoi(argv[7]) != 0;
  const int64_t planes = atoll(argv[8]);
  const size_t bytes = (size_t)(nx * ny * nz) * sizeof(float);
  // dual volumes of the binary16 variants are half as long
  const bool half = strstr(variant, "_h") != nullptr;
  const size_t dbytes = half ? bytes / 2 : bytes;
  Bufs v;
  unsigned seed = 1;
  v.b = guarded(bytes, end_aligned, seed++);
  for (int a = 0; a < 3; ++a) {
    v.p[a] = guarded(dbytes, end_aligned, seed++);
    v.ri[a] = guarded(dbytes, end_aligned, seed++);
    v.ro[a] = guarded(dbytes, end_aligned, seed++);
  }
  v.z = guarded(bytes, end_aligned, seed++);
  for (int a = 0; a < 3; ++a) v.po[a] = guarded(dbytes, end_aligned, seed++);
  if (!strcmp(variant, "fused") || !strcmp(variant, "fused_nostream")) {
    const bool sp = !strcmp(variant, "fused");
    if (wide)
      run_fused<int64_t, uint64_t, float>(v, nx, ny, nz, grid, sp);
    else
      run_fused<int32_t, uint32_t, float>(v, nx, ny, nz, grid, sp);
  } else if (!strcmp(variant, "tb3") || !strcmp(variant, "tb3_h")) {
    if (half) {
      if (wide)
        run_tb3<int64_t, uint64_t, _Float16>(v, nx, ny, nz, grid, planes);
      else
        run_tb3<int32_t, uint32_t, _Float16>(v, nx, ny, nz, grid, planes);
    } else {
      if (wide)
        run_tb3<int64_t, uint64_t, float>(v, nx, ny, nz, grid, planes);
      else
        run_tb3<int32_t, uint32_t, float>(v, nx, ny, nz, grid, planes);
    }
  } else if (!strcmp(variant, "tb2") || !strcmp(variant, "tb2_h")) {
    if (half) {
      if (wide)
        run_tb2<int64_t, uint64_t, _Float16>(v, nx, ny, nz, grid, planes);
      else
        run_tb2<int32_t, uint32_t, _Float16>(v, nx, ny, nz, grid, planes);
    } else {
      if (wide)
        run_tb2<int64_t, uint64_t, float>(v, nx, ny, nz, grid, planes);
      else
        run_tb2<int32_t, uint32_t, float>(v, nx, ny, nz, grid, planes);
    }
  } else if (!strncmp(variant, "pair", 4)) {
    const bool sp = strstr(variant, "nostream") == nullptr;
    if (nx % 2 != 0) {
      printf("ok %s skipped: nx odd\n", variant);
      return 0;
    }
    if (half) {
      if (wide)
        run_pair<int64_t, uint64_t, _Float16>(v, nx, ny, nz, grid, sp);
      else
        run_pair<int32_t, uint32_t, _Float16>(v, nx, ny, nz, grid, sp);
    } else {
      if (wide)
        run_pair<int64_t, uint64_t, float>(v, nx, ny, nz, grid, sp);
      else
        run_pair<int32_t, uint32_t, float>(v, nx, ny, nz, grid, sp);
    }
  } else if (!strcmp(variant, "fused_h") || !strcmp(variant, "fused_nostream_h")) {
    const bool sp = !strcmp(variant, "fused_h");
    if (wide)
      run_fused<int64_t, uint64_t, _Float16>(v, nx, ny, nz, grid, sp);
    else
      run_fused<int32_t, uint32_t, _Float16>(v, nx, ny, nz, grid, sp);
  } else if (wide) {
    run_ablation<int64_t>(variant, v, nx, ny, nz, grid, planes);
  } else {
    run_ablation<int32_t>(variant, v, nx, ny, nz, grid, planes);
  }
  printf("ok %s %lldx%lldx%lld wide=%d grid=%u end=%d planes=%lld\n", variant, (long long)nx,
         (long long)ny, (long long)nz, (int)wide, grid, (int)end_aligned, (long long)planes);
  return 0;
}
