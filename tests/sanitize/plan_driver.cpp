// Test driver for the host planner under AddressSanitizer and
// UndefinedBehaviorSanitizer (CPU only; built with g++, no GPU code).
//
// Reads cases from stdin, one per line:
//   case <grad_dtype> <comm_dtype> <cap_bytes> <first_bytes> <world_size> <map_path|-> <n_params> <numel>...
// and writes one JSON object per case to stdout: the status of
// ddp_bucket_plan_ex, every bucket with its members (from the accessors), the
// arena size and offsets; if map_path is not "-", the arena map is written
// there as raw uint16. Every plan is then freed. After the cases, the error
// paths of every accessor are exercised; the line "errors ok" reports that
// each returned its error status with a message.
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <string>
#include <vector>

#include "ddp_internal.h"

// The device tables exist only in the HIP build; a plan built on the CPU never
// has any.
namespace ddp {
void release_device_tables(ddp_plan*) {}
}  // namespace ddp

namespace {

bool check(bool ok, const char* what) {
  if (!ok) std::fprintf(stderr, "driver: %s\n", what);
  return ok;
}

bool error_paths() {
  bool ok = true;
  ddp_plan* p = nullptr;
  const int64_t numels[3] = {4, 100, 7};
  const int64_t bad[2] = {4, -1};
  auto failed = [](int st) { return st != DDP_OK && ddp_last_error()[0] != '\0'; };
  ok &= check(failed(ddp_bucket_plan(bad, 2, DDP_FP32, 1024, 1024, 1, &p)), "negative numel accepted");
  ok &= check(failed(ddp_bucket_plan(numels, 3, 7, 1024, 1024, 1, &p)), "unknown dtype accepted");
  ok &= check(failed(ddp_bucket_plan(numels, 3, DDP_FP32, 0, 1024, 1, &p)), "zero capacity accepted");
  ok &= check(failed(ddp_bucket_plan(numels, 3, DDP_FP32, 1024, 1024, 65, &p)), "65 ranks accepted");
  ok &= check(failed(ddp_bucket_plan(numels, 3, DDP_FP32, 1024, 1024, 1, nullptr)), "NULL out accepted");
  ok &= check(failed(ddp_bucket_plan(nullptr, 3, DDP_FP32, 1024, 1024, 1, &p)), "NULL numels accepted");
  ok &= check(failed(ddp_bucket_plan_ex(numels, 3, DDP_BF16, DDP_FP32, 1024, 1024, 1, &p)), "bf16->fp32 accepted");
  if (!check(ddp_bucket_plan(numels, 3, DDP_FP32, 64, 32, 2, &p) == DDP_OK, "valid plan refused")) return false;
  int32_t nb = 0, nm = 0, pi = 0;
  int64_t padded = 0, off = 0, m = 0, an = 0;
  ok &= check(ddp_plan_num_buckets(p, &nb) == DDP_OK && nb > 0, "num_buckets");
  ok &= check(failed(ddp_plan_num_buckets(nullptr, &nb)), "num_buckets(NULL)");
  ok &= check(failed(ddp_plan_bucket(p, nb, &padded, &nm)), "bucket index past the end");
  ok &= check(failed(ddp_plan_bucket(p, -1, &padded, &nm)), "negative bucket index");
  ok &= check(failed(ddp_plan_member(p, 0, 1000, &pi, &off, &m)), "member index past the end");
  ok &= check(failed(ddp_plan_member(p, nb, 0, &pi, &off, &m)), "member of a missing bucket");
  ok &= check(failed(ddp_plan_grad_arena(p, nullptr, nullptr)), "grad_arena(NULL)");
  ok &= check(ddp_plan_grad_arena(p, &an, nullptr) == DDP_OK, "grad_arena");
  std::vector<uint16_t> map(size_t(an / 4) + 1);
  ok &= check(failed(ddp_plan_arena_map(p, map.data(), an / 4 + 1)), "arena map of the wrong length");
  ok &= check(ddp_plan_arena_map(p, map.data(), an / 4) == DDP_OK, "arena map");
  ddp_plan_free(p);
  ddp_plan_free(nullptr);
  return ok;
}

}  // namespace

int main() {
  std::string tag;
  while (std::cin >> tag) {
    if (tag != "case") {
      std::fprintf(stderr, "driver: unexpected token %s\n", tag.c_str());
      return 2;
    }
    int32_t gdt, cdt, n, np;
    int64_t cap, first;
    std::string map_path;
    std::cin >> gdt >> cdt >> cap >> first >> n >> map_path >> np;
    std::vector<int64_t> numels(size_t(np > 0 ? np : 1), 0);
    for (int32_t i = 0; i < np; ++i) std::cin >> numels[size_t(i)];
    ddp_plan* p = nullptr;
    const int st = ddp_bucket_plan_ex(numels.data(), np, gdt, cdt, cap, first, n, &p);
    std::printf("{\"status\": %d", st);
    if (st == DDP_OK) {
      int32_t nb = 0;
      ddp_plan_num_buckets(p, &nb);
      std::printf(", \"buckets\": [");
      for (int32_t b = 0; b < nb; ++b) {
        int64_t padded = 0;
        int32_t nm = 0;
        ddp_plan_bucket(p, b, &padded, &nm);
        std::printf("%s{\"padded_numel\": %lld, \"members\": [", b ? ", " : "", (long long)padded);
        for (int32_t i = 0; i < nm; ++i) {
          int32_t pi = 0;
          int64_t off = 0, m = 0;
          ddp_plan_member(p, b, i, &pi, &off, &m);
          std::printf("%s[%d, %lld, %lld]", i ? ", " : "", pi, (long long)off, (long long)m);
        }
        std::printf("]}");
      }
      int64_t an = 0;
      std::vector<int64_t> offs(size_t(np > 0 ? np : 1), -1);
      ddp_plan_grad_arena(p, &an, offs.data());
      std::printf("], \"arena_numel\": %lld, \"offsets\": [", (long long)an);
      for (int32_t i = 0; i < np; ++i) std::printf("%s%lld", i ? ", " : "", (long long)offs[size_t(i)]);
      std::printf("]");
      if (map_path != "-") {
        const int64_t nv = an / (16 / (gdt == DDP_BF16 ? 2 : 4));
        std::vector<uint16_t> map(size_t(nv > 0 ? nv : 1));
        const int mst = ddp_plan_arena_map(p, map.data(), nv);
        std::printf(", \"map_status\": %d", mst);
        if (mst == DDP_OK) {
          FILE* f = std::fopen(map_path.c_str(), "wb");
          if (f == nullptr || std::fwrite(map.data(), sizeof(uint16_t), size_t(nv), f) != size_t(nv)) return 3;
          std::fclose(f);
        }
      }
      ddp_plan_free(p);
    }
    std::printf("}\n");
  }
  std::printf(error_paths() ? "errors ok\n" : "errors FAILED\n");
  return 0;
}
