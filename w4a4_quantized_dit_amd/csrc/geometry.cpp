// DeltaQuant cube geometry on the host ("DeltaQuant on MiniMax-H3", sections "The audio win has
// a mechanism": non-video rows form 1-D cubes of consecutive rows; "Standing configuration": the
// video grid is derived per request and the cube sequence is fixed for a given grid; "Deviations
// from the paper, and one replication": uniform cube-64, a per-timestep cube schedule and
// divisor-aligned cube shapes).
//
// Rows: [n_text | T·H·W video, raster (t, h, w) | n_audio].  Cube ids follow the first row of
// each cube: text cubes, then video cubes in raster order of their (t/ct, h/ch, w/cw)
// coordinates (the first member of such a cube is its corner (t0, h0, w0), and raster order of
// corners is raster order of cube coordinates), then audio cubes.
#include <stdint.h>

#include <vector>

namespace svdq {

int64_t cube_count(int64_t T, int64_t H, int64_t W, int64_t ct, int64_t ch, int64_t cw,
                   int64_t n_text, int64_t n_audio, int64_t c1) {
  const int64_t nt = (T + ct - 1) / ct, nh = (H + ch - 1) / ch, nw = (W + cw - 1) / cw;
  return (n_text + c1 - 1) / c1 + nt * nh * nw + (n_audio + c1 - 1) / c1;
}

void cube_geometry_fill(int64_t T, int64_t H, int64_t W, int64_t ct, int64_t ch, int64_t cw,
                        int64_t n_text, int64_t n_audio, int64_t c1, int32_t* row_to_cube,
                        int32_t* cube_ptr, int32_t* cube_rows) {
  const int64_t nh = (H + ch - 1) / ch, nw = (W + cw - 1) / cw, nt = (T + ct - 1) / ct;
  const int64_t text_cubes = (n_text + c1 - 1) / c1;
  const int64_t video_cubes = nt * nh * nw;
  const int64_t n_cubes = text_cubes + video_cubes + (n_audio + c1 - 1) / c1;
  const int64_t M = n_text + T * H * W + n_audio;
  int64_t m = 0;
  for (int64_t i = 0; i < n_text; ++i) row_to_cube[m++] = (int32_t)(i / c1);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t w = 0; w < W; ++w)
        row_to_cube[m++] = (int32_t)(text_cubes + ((t / ct) * nh + h / ch) * nw + w / cw);
  for (int64_t i = 0; i < n_audio; ++i)
    row_to_cube[m++] = (int32_t)(text_cubes + video_cubes + i / c1);
  // counting sort of rows by cube id keeps members ascending
  std::vector<int64_t> count(n_cubes + 1, 0);
  for (int64_t i = 0; i < M; ++i) ++count[row_to_cube[i] + 1];
  cube_ptr[0] = 0;
  for (int64_t c = 0; c < n_cubes; ++c) cube_ptr[c + 1] = (int32_t)(cube_ptr[c] + count[c + 1]);
  std::vector<int64_t> fill(cube_ptr, cube_ptr + n_cubes);
  for (int64_t i = 0; i < M; ++i) cube_rows[fill[row_to_cube[i]]++] = (int32_t)i;
}

// Largest divisor of n not above e (n <= 0: e itself).
int64_t divisor_edge(int64_t n, int64_t e) {
  if (n <= 0) return e;
  for (int64_t d = e < n ? e : n; d > 1; --d)
    if (n % d == 0) return d;
  return 1;
}

// Greedy packing of consecutive cubes into the activation kernel's work groups: a group takes
// cubes while it holds at most max_rows rows and max_cubes cubes.  Returns the number of groups,
// or -1 when a cube is larger than max_rows (or empty).
int64_t cube_groups(const int32_t* cube_ptr, int64_t n_cubes, int64_t max_rows,
                    int64_t max_cubes, int32_t* group_ptr) {
  int64_t g = 0, rows = 0, cubes = 0;
  if (group_ptr) group_ptr[0] = 0;
  for (int64_t c = 0; c < n_cubes; ++c) {
    const int64_t n = (int64_t)cube_ptr[c + 1] - cube_ptr[c];
    if (n < 1 || n > max_rows) return -1;
    if (cubes > 0 && (rows + n > max_rows || cubes + 1 > max_cubes)) {
      ++g;
      if (group_ptr) group_ptr[g] = (int32_t)c;
      rows = 0;
      cubes = 0;
    }
    rows += n;
    ++cubes;
  }
  if (n_cubes > 0) ++g;
  if (group_ptr) group_ptr[g] = (int32_t)n_cubes;
  return g;
}

}  // namespace svdq
