// CPU functional emulation of the HIP kernels (test infrastructure).
//
// The kernel headers are compiled as host C++ with the shim in threaded mode:
// every thread of a workgroup runs as an OS thread and __syncthreads() is a
// real barrier over them, so data exchanged through LDS (a static array here,
// shared by the workgroup's threads; workgroups run one after another) behaves
// as on the GPU.  Arithmetic is IEEE binary32 with no contraction, as on the
// GPU, so results can be compared bit for bit with the CPU oracle.
//
// usage: func <kernel> <nx> <ny> <nz> <lambda> <m1> <m2> <dir> <wide:0|1> <grid:0=as launched>
//             [planes: tb2 slab length, 0 = as launched]
//   kernel: fused  one step (m1), p updated in place
//           cube, cube_8x8x8  one step (m1) with the cube-tiled kernel
//           lds_march  one step (m1) with the LDS z-march (64 x 4 tiles, 8 planes)
//           lds_march_<TX>x<TY>  the same with TX x TY tiles (32x4, 32x8, 32x16, 64x8)
//           gap    duality gap of p (three doubles written to <dir>/gap.bin)
//           gap_pair  the same with two voxels per lane (even nx)
//           pair   one step of the two-voxels-per-lane kernel (even nx)
//           pair_h the same with p and r stored as binary16
//           tb2    two steps (m1 then m2) in one pass, p_in -> p_out
//           tb2_h  the same with p and r stored as binary16 (files hold the
//                  binary16 values as floats)
//           tb3, tb3_h  three steps (m1, m2, m3) in one pass
//   dir holds b.bin (n floats), p.bin and r.bin (3n floats each); the kernel
//   writes p_out.bin and r_out.bin there.
#include <condition_variable>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <string>
#include <thread>
#include <vector>

#include "tv_fgp_fused_kernel.hpp"
#include "tv_fgp_tb2_kernel.hpp"
#include "tv_fgp_tb3_kernel.hpp"
#include "tv_fgp_cube_kernel.hpp"
#include "tv_fgp_lds_kernel.hpp"
#include "tv_fgp_gap_kernel.hpp"
#include "tv_fgp_pair_kernel.hpp"

thread_local EmulDim3 threadIdx, blockIdx, gridDim, blockDim;

namespace {

// A workgroup barrier as the hardware's: it waits for the threads that have
// not yet ended (a thread that returns leaves it).
struct Barrier {
  std::mutex mu;
  std::condition_variable cv;
  unsigned count = 0, waiting = 0, generation = 0;
  void release() {
    waiting = 0;
    ++generation;
    cv.notify_all();
  }
  void wait() {
    std::unique_lock<std::mutex> lock(mu);
    const unsigned gen = generation;
    if (++waiting == count) {
      release();
    } else {
      cv.wait(lock, [&] { return gen != generation; });
    }
  }
  void leave() {
    std::unique_lock<std::mutex> lock(mu);
    --count;
    if (waiting > 0 && waiting == count) release();
  }
};

Barrier g_barrier;

}  // namespace

void emul_syncthreads() { g_barrier.wait(); }

namespace {

template <typename F>
void run_grid(unsigned grid, unsigned block, F &&body) {
  for (unsigned bl = 0; bl < grid; ++bl) {
    g_barrier.count = block;
    std::vector<std::thread> threads;
    threads.reserve(block);
    for (unsigned th = 0; th < block; ++th) {
      threads.emplace_back([&, bl, th] {
        gridDim = {grid, 1, 1};
        blockDim = {block, 1, 1};
        blockIdx = {bl, 0, 0};
        threadIdx = {th, 0, 0};
        body();
        g_barrier.leave();
      });
    }
    for (auto &t : threads) t.join();
  }
}

std::vector<float> read_file(const std::string &path, size_t n) {
  std::vector<float> v(n);
  FILE *f = fopen(path.c_str(), "rb");
  if (!f || fread(v.data(), sizeof(float), n, f) != n) {
    fprintf(stderr, "cannot read %s\n", path.c_str());
    exit(3);
  }
  fclose(f);
  return v;
}

void write_file(const std::string &path, const std::vector<float> &v) {
  FILE *f = fopen(path.c_str(), "wb");
  if (!f || fwrite(v.data(), sizeof(float), v.size(), f) != v.size()) {
    fprintf(stderr, "cannot write %s\n", path.c_str());
    exit(3);
  }
  fclose(f);
}

unsigned pick(int64_t ntiles, unsigned grid) {
  return grid ? grid : tvfgp::grid_for(ntiles);
}

template <typename I, int TX, int TY>
void run_march(int64_t nx, int64_t ny, int64_t nz, int64_t planes, unsigned grid,
               const float *b, float *p, const float *r, float *r_out, float lam, float c,
               float m) {
  const size_t n = (size_t)(nx * ny * nz);
  const tvfgp::Geometry<I> g = tvfgp::march_geometry<I>(nx, ny, nz, planes, TX, TY);
  run_grid(pick(g.ntiles, grid), TX * TY, [&] {
    tvfgp::lds_march_kernel<I, TX, TY>(b, p, p + n, p + 2 * n, r, r + n, r + 2 * n, r_out,
                                       r_out + n, r_out + 2 * n, lam, c, m, g);
  });
}

template <typename I, typename Off>
void run(const char *kernel, int64_t nx, int64_t ny, int64_t nz, float lam, float m1, float m2,
         float m3,
         unsigned grid, const float *b, float *p, float *r, float *p_out, float *r_out,
         const std::string &dir, int64_t planes) {
  const size_t n = (size_t)(nx * ny * nz);
  const float c = 1.0f / (12.0f * lam);
  if (!strcmp(kernel, "fused")) {
    const auto g = tvfgp::zx_geometry<I, Off>(nx, ny, nz);
    run_grid(pick(g.ntiles, grid), tvfgp::kZxBlock, [&] {
      tvfgp::fused_zx_kernel<I, Off, true, float>(b, p, p + n, p + 2 * n, r, r + n, r + 2 * n,
                                                  r_out, r_out + n, r_out + 2 * n, lam, c, m1,
                                                  g);
    });
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "pair")) {
    if (nx % 2 != 0) {
      fprintf(stderr, "pair needs an even nx\n");
      exit(2);
    }
    const auto g = tvfgp::pair_geometry<I, Off>(nx, ny, nz);
    run_grid(pick(g.ntiles, grid), tvfgp::kPairBlock, [&] {
      tvfgp::fused_pair_kernel<I, Off, true, float>(b, p, p + n, p + 2 * n, r, r + n,
                                                    r + 2 * n, r_out, r_out + n,
                                                    r_out + 2 * n, lam, c, m1, g);
    });
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "pair_h")) {
    // binary16 dual: the inputs must be binary16 values (converted exactly)
    if (nx % 2 != 0) {
      fprintf(stderr, "pair_h needs an even nx\n");
      exit(2);
    }
    typedef _Float16 h;
    std::vector<h> ph(3 * n), rh(3 * n), roh(3 * n);
    for (size_t i = 0; i < 3 * n; ++i) {
      ph[i] = (h)p[i];
      rh[i] = (h)r[i];
    }
    const auto g = tvfgp::pair_geometry<I, Off>(nx, ny, nz);
    h *P = ph.data(), *R = rh.data(), *RO = roh.data();
    run_grid(pick(g.ntiles, grid), tvfgp::kPairBlock, [&] {
      tvfgp::fused_pair_kernel<I, Off, true, h>(b, P, P + n, P + 2 * n, R, R + n, R + 2 * n,
                                                RO, RO + n, RO + 2 * n, lam, c, m1, g);
    });
    for (size_t i = 0; i < 3 * n; ++i) {
      p_out[i] = (float)ph[i];
      r_out[i] = (float)roh[i];
    }
  } else if (!strcmp(kernel, "gap") || !strcmp(kernel, "gap_pair")) {
    // duality gap of p: the three sums go to <dir>/gap.bin as doubles
    const bool pair = !strcmp(kernel, "gap_pair");
    if (pair && nx % 2 != 0) {
      fprintf(stderr, "gap_pair needs an even nx\n");
      exit(2);
    }
    const int count = grid ? (int)grid
                           : pair ? tvfgp::gap_pair_grid(nx, ny, nz) : tvfgp::gap_grid(nx, ny, nz);
    std::vector<double> partial((size_t)count * 3);
    if (pair) {
      const auto g = tvfgp::gap_pair_geometry<I, Off>(nx, ny, nz);
      run_grid((unsigned)count, tvfgp::kPairBlock, [&] {
        tvfgp::gap_partial_pair_kernel<I, Off>(b, p, p + n, p + 2 * n, lam, g, partial.data());
      });
    } else {
      const auto g = tvfgp::zx_geometry<I, Off>(nx, ny, nz);
      run_grid((unsigned)count, tvfgp::kZxBlock, [&] {
        tvfgp::gap_partial_kernel<I, Off>(b, p, p + n, p + 2 * n, lam, g, partial.data());
      });
    }
    double out[3];
    run_grid(1, tvfgp::kGapFinalBlock,
             [&] { tvfgp::gap_final_kernel(partial.data(), count, (double)lam, out); });
    FILE *f = fopen((dir + "/gap.bin").c_str(), "wb");
    if (!f || fwrite(out, sizeof(double), 3, f) != 3) {
      fprintf(stderr, "cannot write gap.bin\n");
      exit(3);
    }
    fclose(f);
  } else if (!strcmp(kernel, "lds_march")) {
    run_march<I, tvfgp::kTileX, tvfgp::kTileY>(nx, ny, nz, planes > 0 ? planes : 8, grid, b, p, r,
                                               r_out, lam, c, m1);
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "lds_march_32x4")) {
    run_march<I, 32, 4>(nx, ny, nz, planes > 0 ? planes : 8, grid, b, p, r, r_out, lam, c, m1);
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "lds_march_32x8")) {
    run_march<I, 32, 8>(nx, ny, nz, planes > 0 ? planes : 8, grid, b, p, r, r_out, lam, c, m1);
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "lds_march_32x16")) {
    run_march<I, 32, 16>(nx, ny, nz, planes > 0 ? planes : 8, grid, b, p, r, r_out, lam, c, m1);
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "lds_march_64x8")) {
    run_march<I, 64, 8>(nx, ny, nz, planes > 0 ? planes : 8, grid, b, p, r, r_out, lam, c, m1);
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "cube")) {
    const auto g = tvfgp::cube_geometry<I, 16, 8, 4>(nx, ny, nz);
    run_grid(pick(g.ntiles, grid), tvfgp::kCubeBlock, [&] {
      tvfgp::cube_kernel<I, 16, 8, 4>(b, p, p + n, p + 2 * n, r, r + n, r + 2 * n, r_out,
                                      r_out + n, r_out + 2 * n, lam, c, m1, g);
    });
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "cube_8x8x8")) {
    const auto g = tvfgp::cube_geometry<I, 8, 8, 8>(nx, ny, nz);
    run_grid(pick(g.ntiles, grid), tvfgp::kCubeBlock, [&] {
      tvfgp::cube_kernel<I, 8, 8, 8>(b, p, p + n, p + 2 * n, r, r + n, r + 2 * n, r_out,
                                     r_out + n, r_out + 2 * n, lam, c, m1, g);
    });
    memcpy(p_out, p, 3 * n * sizeof(float));
  } else if (!strcmp(kernel, "tb3")) {
    const auto g = tvfgp::tb_geometry<I, Off>(nx, ny, nz,
                                              planes > 0 ? planes : tvfgp::tb3_planes(nx, ny, nz));
    run_grid(pick(g.ntiles, grid), tvfgp::kTbBlock, [&] {
      tvfgp::tb3_kernel<I, Off, float>(b, p, p + n, p + 2 * n, p_out, p_out + n, p_out + 2 * n,
                                       r, r + n, r + 2 * n, r_out, r_out + n, r_out + 2 * n, lam,
                                       c, m1, m2, m3, g);
    });
  } else if (!strcmp(kernel, "tb3_h")) {
    typedef _Float16 h;
    std::vector<h> ph(3 * n), rh(3 * n), poh(3 * n), roh(3 * n);
    for (size_t i = 0; i < 3 * n; ++i) {
      ph[i] = (h)p[i];
      rh[i] = (h)r[i];
    }
    const auto g = tvfgp::tb_geometry<I, Off>(nx, ny, nz,
                                              planes > 0 ? planes : tvfgp::tb3_planes(nx, ny, nz));
    h *P = ph.data(), *R = rh.data(), *PO = poh.data(), *RO = roh.data();
    run_grid(pick(g.ntiles, grid), tvfgp::kTbBlock, [&] {
      tvfgp::tb3_kernel<I, Off, h>(b, P, P + n, P + 2 * n, PO, PO + n, PO + 2 * n, R, R + n,
                                   R + 2 * n, RO, RO + n, RO + 2 * n, lam, c, m1, m2, m3, g);
    });
    for (size_t i = 0; i < 3 * n; ++i) {
      p_out[i] = (float)poh[i];
      r_out[i] = (float)roh[i];
    }
  } else if (!strcmp(kernel, "tb2")) {
    const auto g = tvfgp::tb_geometry<I, Off>(nx, ny, nz, planes);
    run_grid(pick(g.ntiles, grid), tvfgp::kTbBlock, [&] {
      tvfgp::tb2_kernel<I, Off, float>(b, p, p + n, p + 2 * n, p_out, p_out + n, p_out + 2 * n,
                                       r, r + n, r + 2 * n, r_out, r_out + n, r_out + 2 * n, lam,
                                       c, m1, m2, g);
    });
  } else if (!strcmp(kernel, "tb2_h")) {
    // binary16 dual: the inputs must be binary16 values (converted exactly)
    typedef _Float16 h;
    std::vector<h> ph(3 * n), rh(3 * n), poh(3 * n), roh(3 * n);
    for (size_t i = 0; i < 3 * n; ++i) {
      ph[i] = (h)p[i];
      rh[i] = (h)r[i];
    }
    const auto g = tvfgp::tb_geometry<I, Off>(nx, ny, nz, planes);
    h *P = ph.data(), *R = rh.data(), *PO = poh.data(), *RO = roh.data();
    run_grid(pick(g.ntiles, grid), tvfgp::kTbBlock, [&] {
      tvfgp::tb2_kernel<I, Off, h>(b, P, P + n, P + 2 * n, PO, PO + n, PO + 2 * n, R, R + n,
                                   R + 2 * n, RO, RO + n, RO + 2 * n, lam, c, m1, m2, g);
    });
    for (size_t i = 0; i < 3 * n; ++i) {
      p_out[i] = (float)poh[i];
      r_out[i] = (float)roh[i];
    }
  } else {
    fprintf(stderr, "unknown kernel %s\n", kernel);
    exit(2);
  }
}

}  // namespace

int main(int argc, char **argv) {
  // func slabs nx ny nz slots: the slab lengths the multi-step launchers pick
  if (argc == 6 && !strcmp(argv[1], "slabs")) {
    const int64_t nx = atoll(argv[2]), ny = atoll(argv[3]), nz = atoll(argv[4]);
    printf("%lld %lld\n", (long long)tvfgp::tb3_planes(nx, ny, nz, atoll(argv[5])),
           (long long)tvfgp::tb_planes(nx, ny, nz));
    return 0;
  }
  if (argc < 11 || argc > 13) {
    fprintf(stderr, "usage: func kernel nx ny nz lambda m1 m2 dir wide grid [planes [m3]]\n");
    return 2;
  }
  const int64_t planes = argc >= 12 ? atoll(argv[11]) : 0;
  const float m3 = argc == 13 ? strtof(argv[12], nullptr) : 0.0f;
  const char *kernel = argv[1];
  const int64_t nx = atoll(argv[2]), ny = atoll(argv[3]), nz = atoll(argv[4]);
  const float lam = strtof(argv[5], nullptr), m1 = strtof(argv[6], nullptr),
              m2 = strtof(argv[7], nullptr);
  const std::string dir = argv[8];
  const bool wide = atoi(argv[9]) != 0;
  const unsigned grid = (unsigned)atoi(argv[10]);
  const size_t n = (size_t)(nx * ny * nz);
  std::vector<float> b = read_file(dir + "/b.bin", n);
  std::vector<float> p = read_file(dir + "/p.bin", 3 * n);
  std::vector<float> r = read_file(dir + "/r.bin", 3 * n);
  std::vector<float> p_out(3 * n, -12345.0f), r_out(3 * n, -12345.0f);
  if (wide)
    run<int64_t, uint64_t>(kernel, nx, ny, nz, lam, m1, m2, m3, grid, b.data(), p.data(),
                           r.data(), p_out.data(), r_out.data(), dir, planes);
  else
    run<int32_t, uint32_t>(kernel, nx, ny, nz, lam, m1, m2, m3, grid, b.data(), p.data(),
                           r.data(), p_out.data(), r_out.data(), dir, planes);
  write_file(dir + "/p_out.bin", p_out);
  write_file(dir + "/r_out.bin", r_out);
  printf("ok %s %lldx%lldx%lld\n", kernel, (long long)nx, (long long)ny, (long long)nz);
  return 0;
}
