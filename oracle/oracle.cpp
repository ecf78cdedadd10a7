// CPU oracle for submanifold sparse 3x3x3 convolution (SubMConv3d) and its k=1 case.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link, load or
// call this file or the library built from it: only the tests, the package smoke
// check and the CPU-baseline leg of the benchmark do.  It shares no code, header,
// table or constant with the HIP library.
//
// What it computes, written straight from the definition, slow and plain:
//
//   * Every SparseConv3d in the TRELLIS.2-lineage models is built with stride 1 and no
//     padding, which makes it a submanifold convolution: the output sites are exactly
//     the input sites (LATO.2 MLX port page, "The scope, once measured").
//   * The reference method there is a dictionary lookup with a per-voxel loop, and the
//     convention it implements is cross-correlation: the tap at offset d reads the
//     feature row of site c + d (LATO.2 MLX port page, "Correctness").
//   * The plain gather-scatter algorithm: build a hash map of the active voxel
//     coordinates, gather the neighbour for each kernel offset, multiply by that
//     offset's weight matrix, accumulate into the original voxel (trellis-mac article,
//     section on replacing the sparse 3D convolution, its flowchart).
//   * Weights are laid out [K^3, Cin, Cout] (Pixal3D MLX port README, "Status": the
//     KRSC -> [K^3, in, out] remap).
//
// Readings taken where the pages are silent (each is listed in the design notes):
//   * taps are numbered t = 9*(dx+1) + 3*(dy+1) + (dz+1), so the centre tap is 13;
//   * a neighbour outside the grid, or in another batch entry, simply is not in the
//     dictionary, so it contributes nothing (zero padding);
//   * coordinates outside [0,batch) x [0,Gx) x [0,Gy) x [0,Gz) are an error (-2), a
//     repeated coordinate is an error (-3);
//   * accumulation is in fp64 from the exact input values.
//
// Build: g++ -O3 -march=x86-64-v3 -fopenmp -shared -fPIC oracle.cpp -o liboracle.so
#include <cstdint>
#include <cstddef>
#include <functional>
#include <unordered_map>
#include <vector>
#include <omp.h>

namespace {

struct Site {
  int32_t b, x, y, z;
  bool operator==(const Site& o) const {
    return b == o.b && x == o.x && y == o.y && z == o.z;
  }
};

struct SiteHash {
  size_t operator()(const Site& s) const {
    // Any hash is correct here: equality on all four fields decides membership.
    size_t h = std::hash<int32_t>()(s.b);
    h = h * 1000003u ^ std::hash<int32_t>()(s.x);
    h = h * 1000003u ^ std::hash<int32_t>()(s.y);
    h = h * 1000003u ^ std::hash<int32_t>()(s.z);
    return h;
  }
};

constexpr int kOk = 0;
constexpr int kErrArg = -1;
constexpr int kErrCoordRange = -2;
constexpr int kErrDuplicate = -3;

}  // namespace

extern "C" {

// Number of OpenMP threads the oracle's parallel loops use.
int oracle_num_threads() { return omp_get_max_threads(); }

// Sets that number (for timing the oracle on one core and on all of them).
void oracle_set_num_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}

// Neighbour map of a set of active sites.
//   coords  [n, 4] int32 rows (b, x, y, z)
//   ksize   3 (27 taps) or 1 (one tap, the site itself)
//   nbr     [n, ksize^3] int32 out: row index of site (b, x+dx, y+dy, z+dz), or -1
// Returns 0, -1 (bad argument), -2 (coordinate out of range) or -3 (duplicate site).
int oracle_build_map(const int32_t* coords, int64_t n, int32_t batch, int32_t gx, int32_t gy,
                     int32_t gz, int32_t ksize, int32_t* nbr) {
  if (n < 0 || (ksize != 1 && ksize != 3)) return kErrArg;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* c = coords + 4 * i;
    if (c[0] < 0 || c[0] >= batch || c[1] < 0 || c[1] >= gx || c[2] < 0 || c[2] >= gy ||
        c[3] < 0 || c[3] >= gz)
      return kErrCoordRange;
  }
  // The dictionary: coordinate -> row.
  std::unordered_map<Site, int64_t, SiteHash> dict;
  dict.reserve(static_cast<size_t>(n) * 2 + 1);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* c = coords + 4 * i;
    if (!dict.emplace(Site{c[0], c[1], c[2], c[3]}, i).second) return kErrDuplicate;
  }
  const int r = ksize / 2;
  const int taps = ksize * ksize * ksize;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* c = coords + 4 * i;
    int t = 0;
    for (int dx = -r; dx <= r; ++dx)
      for (int dy = -r; dy <= r; ++dy)
        for (int dz = -r; dz <= r; ++dz, ++t) {
          auto it = dict.find(Site{c[0], c[1] + dx, c[2] + dy, c[3] + dz});
          nbr[i * taps + t] = (it == dict.end()) ? -1 : static_cast<int32_t>(it->second);
        }
  }
  return kOk;
}

// Submanifold convolution over a neighbour map, fp64:
//   Y[i][o] = bias[o] + sum_t sum_c X[nbr[i][t]][c] * W[t][c][o]   (taps with nbr = -1 skipped)
//   X [n, cin], W [taps, cin, cout], bias [cout] or NULL, nbr [n, taps], Y [n, cout].
// flip = 1 evaluates the other orientation the LATO.2 page leaves open: the tap at
// offset d reads site c - d, i.e. row nbr[i][taps-1-t] is paired with W[t].
void oracle_conv(const double* X, const double* W, const double* bias, const int32_t* nbr,
                 int64_t n, int32_t taps, int32_t cin, int32_t cout, int32_t flip, double* Y) {
#pragma omp parallel
  {
    std::vector<double> acc(static_cast<size_t>(cout));
#pragma omp for schedule(dynamic, 256)
    for (int64_t i = 0; i < n; ++i) {
      for (int32_t o = 0; o < cout; ++o) acc[o] = bias ? bias[o] : 0.0;
      for (int32_t t = 0; t < taps; ++t) {
        const int32_t j = nbr[i * taps + (flip ? taps - 1 - t : t)];
        if (j < 0) continue;
        const double* xr = X + static_cast<int64_t>(j) * cin;
        const double* wt = W + static_cast<int64_t>(t) * cin * cout;
        for (int32_t c = 0; c < cin; ++c) {
          const double xv = xr[c];
          const double* wr = wt + static_cast<int64_t>(c) * cout;
          for (int32_t o = 0; o < cout; ++o) acc[o] += xv * wr[o];
        }
      }
      double* yr = Y + i * cout;
      for (int32_t o = 0; o < cout; ++o) yr[o] = acc[o];
    }
  }
}

// k=1 SubMConv3d = per-voxel linear map, fp64: Y[i][o] = bias[o] + sum_c X[i][c] * W[c][o]
// (LATO.2 MLX port page, "Status": SubMConv3d is tested with k=3 and k=1).
void oracle_linear(const double* X, const double* W, const double* bias, int64_t n, int32_t cin,
                   int32_t cout, double* Y) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double* yr = Y + i * cout;
    for (int32_t o = 0; o < cout; ++o) yr[o] = bias ? bias[o] : 0.0;
    for (int32_t c = 0; c < cin; ++c) {
      const double xv = X[i * cin + c];
      const double* wr = W + static_cast<int64_t>(c) * cout;
      for (int32_t o = 0; o < cout; ++o) yr[o] += xv * wr[o];
    }
  }
}

}  // extern "C"
