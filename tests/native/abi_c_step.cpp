// A C-ABI consumer with no Python and no torch: it drives libfp8z1 through
// include/fp8z1.h with its own HIP allocations and stream.
//
//   abi_c_step <dir> [graph]
//
// <dir>/meta.txt:  n_params dp rank steps
//                  E R C                      (n_params lines)
//                  lr beta1 beta2 eps wd max_grad_norm
//                  loss_scaling init_scale growth_factor backoff_factor growth_interval scale_rule
//                  extra_sumsq                (one line per step)
// <dir>/master_<p>.bin  float32 [E,R,C] for every param
// <dir>/grad_<t>_<p>.bin float32 [E,R,C] for every step t (1-based) and param
// Writes <dir>/out_master.bin (the folded FP32 master shard), out_codes_<p>.bin
// and out_scales_<p>.bin (row-major codes and [E,Rb,Cb] scales after the last
// step; positions the shard does not hold stay 0), out_state.txt.
// The step reads the row-major grads (fp8z1_step_rowmajor).  With "graph"
// (a single rank, extra_sumsq 0): step 1 runs as plain calls -- the
// statistics-only pass, fp8z1_shard_sumsq into a device double, the step
// reading that sum through hp.d_global_sumsq, the unfold -- then the same
// calls are captured once into a HIP graph, and every later step copies its
// grads into the captured buffers and launches the graph.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../include/fp8z1.h"

#define CHECK_HIP(x)                                                                 \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      std::exit(3);                                                                  \
    }                                                                                \
  } while (0)
#define CHECK(x)                                                                     \
  do {                                                                               \
    int rc_ = (x);                                                                   \
    if (rc_ != FP8Z1_OK) {                                                           \
      std::fprintf(stderr, "fp8z1 error %d (%s): %s at %s:%d\n", rc_, fp8z1_status_string(rc_), \
                   fp8z1_last_error(), __FILE__, __LINE__);                          \
      std::exit(4);                                                                  \
    }                                                                                \
  } while (0)

static std::vector<char> read_file(const std::string& path, size_t bytes) {
  std::vector<char> buf(bytes);
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f || std::fread(buf.data(), 1, bytes, f) != bytes) {
    std::fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path.c_str());
    std::exit(2);
  }
  std::fclose(f);
  return buf;
}

static void write_file(const std::string& path, const void* data, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(data, 1, bytes, f) != bytes) std::exit(2);
  std::fclose(f);
}

int main(int argc, char** argv) {
  if (argc != 2 && argc != 3) return 1;
  const std::string dir = argv[1];
  const bool graph = argc == 3 && std::string(argv[2]) == "graph";
  FILE* m = std::fopen((dir + "/meta.txt").c_str(), "r");
  if (!m) return 2;
  int n, dp, rank, steps;
  if (std::fscanf(m, "%d %d %d %d", &n, &dp, &rank, &steps) != 4) return 2;
  std::vector<fp8z1_shape> shapes(n);
  for (auto& s : shapes)
    if (std::fscanf(m, "%ld %ld %ld", &s.E, &s.R, &s.C) != 3) return 2;
  fp8z1_hparams hp{};
  if (std::fscanf(m, "%f %f %f %f %f %f", &hp.lr, &hp.beta1, &hp.beta2, &hp.eps, &hp.weight_decay,
                  &hp.max_grad_norm) != 6)
    return 2;
  if (std::fscanf(m, "%d %f %f %f %d %d", &hp.loss_scaling, &hp.init_scale, &hp.growth_factor, &hp.backoff_factor,
                  &hp.growth_interval, &hp.scale_rule) != 6)
    return 2;
  std::vector<double> extra(steps);
  for (auto& x : extra)
    if (std::fscanf(m, "%lf", &x) != 1) return 2;
  std::fclose(m);

  fp8z1_table* table = nullptr;
  CHECK(fp8z1_build_table(shapes.data(), n, dp, rank, FP8Z1_SPLIT_BLOCK, &table));
  fp8z1_table_info info;
  CHECK(fp8z1_table_info_get(table, &info));
  const size_t slots = static_cast<size_t>(info.shard_slots), el = slots * 16384;

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  float *master, *mom1, *mom2;
  uint8_t* fp8;
  float* scales;
  double* ws;
  double* glob;
  fp8z1_state* state;
  size_t wsb = 0;
  CHECK(fp8z1_step_workspace_bytes(table, &wsb));
  CHECK_HIP(hipMalloc(&master, el * 4));
  CHECK_HIP(hipMalloc(&mom1, el * 4));
  CHECK_HIP(hipMalloc(&mom2, el * 4));
  CHECK_HIP(hipMalloc(&fp8, el));
  CHECK_HIP(hipMalloc(&scales, slots * 4 + 4));
  CHECK_HIP(hipMalloc(&ws, wsb + 8));
  CHECK_HIP(hipMalloc(&glob, sizeof(double)));
  CHECK_HIP(hipMalloc(&state, sizeof(fp8z1_state)));
  CHECK_HIP(hipMemset(mom1, 0, el * 4));
  CHECK_HIP(hipMemset(mom2, 0, el * 4));

  std::vector<void*> params(n), grads(n), codes(n), pscales(n);
  std::vector<size_t> nel(n), nsc(n);
  for (int p = 0; p < n; ++p) {
    nel[p] = static_cast<size_t>(shapes[p].E * shapes[p].R * shapes[p].C);
    nsc[p] = static_cast<size_t>(shapes[p].E * ((shapes[p].R + 127) / 128) * ((shapes[p].C + 127) / 128));
    CHECK_HIP(hipMalloc(&params[p], nel[p] * 4));
    CHECK_HIP(hipMalloc(&grads[p], nel[p] * 4));
    CHECK_HIP(hipMalloc(&codes[p], nel[p]));
    CHECK_HIP(hipMalloc(&pscales[p], nsc[p] * 4));
    CHECK_HIP(hipMemset(codes[p], 0, nel[p]));
    CHECK_HIP(hipMemset(pscales[p], 0, nsc[p] * 4));
    auto h = read_file(dir + "/master_" + std::to_string(p) + ".bin", nel[p] * 4);
    CHECK_HIP(hipMemcpy(params[p], h.data(), nel[p] * 4, hipMemcpyHostToDevice));
  }

  CHECK(fp8z1_fold(table, const_cast<const void* const*>(params.data()), FP8Z1_F32, master, nullptr, stream));
  CHECK(fp8z1_state_init(&hp, state, stream));
  const void* const* gl = const_cast<const void* const*>(grads.data());
  float* const* sl = reinterpret_cast<float* const*>(pscales.data());
  // one step of the device-statistics sequence (graph mode)
  fp8z1_hparams hpg = hp;
  hpg.d_global_sumsq = glob;
  auto device_stats_step = [&]() {
    CHECK(fp8z1_fold(table, gl, FP8Z1_F32, nullptr, ws, stream));
    CHECK(fp8z1_shard_sumsq(table, ws, glob, stream));
    CHECK(fp8z1_step_rowmajor(table, &hpg, state, gl, master, mom1, mom2, fp8, scales, nullptr, 0, stream));
    CHECK(fp8z1_unfold(table, fp8, FP8Z1_E4M3, scales, codes.data(), sl, stream));
  };
  hipGraphExec_t exec = nullptr;
  for (int t = 1; t <= steps; ++t) {
    for (int p = 0; p < n; ++p) {
      auto h = read_file(dir + "/grad_" + std::to_string(t) + "_" + std::to_string(p) + ".bin", nel[p] * 4);
      CHECK_HIP(hipMemcpyAsync(grads[p], h.data(), nel[p] * 4, hipMemcpyHostToDevice, stream));
      CHECK_HIP(hipStreamSynchronize(stream));
    }
    if (!graph) {
      hp.extra_sumsq = extra[t - 1];
      CHECK(fp8z1_step_rowmajor(table, &hp, state, gl, master, mom1, mom2, fp8, scales, ws, wsb, stream));
      CHECK(fp8z1_unfold(table, fp8, FP8Z1_E4M3, scales, codes.data(), sl, stream));
    } else if (t == 1) {
      device_stats_step();  // sets the table up and uploads these pointer lists
      CHECK_HIP(hipStreamSynchronize(stream));
      hipGraph_t g;
      CHECK_HIP(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
      device_stats_step();
      CHECK_HIP(hipStreamEndCapture(stream, &g));
      CHECK_HIP(hipGraphInstantiate(&exec, g, nullptr, nullptr, 0));
      CHECK_HIP(hipGraphDestroy(g));
    } else {
      CHECK_HIP(hipGraphLaunch(exec, stream));
      CHECK_HIP(hipStreamSynchronize(stream));
    }
  }
  if (exec) CHECK_HIP(hipGraphExecDestroy(exec));
  fp8z1_state st;
  CHECK(fp8z1_state_read(state, &st, stream));

  std::vector<char> hm(el * 4);
  CHECK_HIP(hipMemcpy(hm.data(), master, el * 4, hipMemcpyDeviceToHost));
  write_file(dir + "/out_master.bin", hm.data(), el * 4);
  for (int p = 0; p < n; ++p) {
    std::vector<char> hc(nel[p]), hs(nsc[p] * 4);
    CHECK_HIP(hipMemcpy(hc.data(), codes[p], nel[p], hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hs.data(), pscales[p], nsc[p] * 4, hipMemcpyDeviceToHost));
    write_file(dir + "/out_codes_" + std::to_string(p) + ".bin", hc.data(), nel[p]);
    write_file(dir + "/out_scales_" + std::to_string(p) + ".bin", hs.data(), nsc[p] * 4);
    CHECK_HIP(hipFree(params[p]));
    CHECK_HIP(hipFree(grads[p]));
    CHECK_HIP(hipFree(codes[p]));
    CHECK_HIP(hipFree(pscales[p]));
  }
  FILE* so = std::fopen((dir + "/out_state.txt").c_str(), "w");
  std::fprintf(so, "%ld %.17g %d %d\n", static_cast<long>(st.step), static_cast<double>(st.k), st.found_inf,
               st.skipped_total);
  std::fclose(so);
  fp8z1_table_free(table);
  CHECK_HIP(hipFree(master));
  CHECK_HIP(hipFree(mom1));
  CHECK_HIP(hipFree(mom2));
  CHECK_HIP(hipFree(fp8));
  CHECK_HIP(hipFree(scales));
  CHECK_HIP(hipFree(ws));
  CHECK_HIP(hipFree(glob));
  CHECK_HIP(hipFree(state));
  CHECK_HIP(hipStreamDestroy(stream));
  std::printf("abi_c_step ok: %zu slots, %d steps%s\n", slots, steps, graph ? ", graph" : "");
  return 0;
}
