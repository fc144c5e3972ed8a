// Host-only driver for the planner under AddressSanitizer and
// UndefinedBehaviorSanitizer: builds a plan from each argument quadruple
// (irreps_x, irreps_y, irreps_out, "mode/select/collapse") and prints the
// status, or the plan's sizes, one line per case. Only the planner (plan.cpp)
// is linked; the four device-table release functions it calls on teardown
// belong to kernel translation units and have nothing to release here.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "common.hpp"

namespace cgtp {
void free_uvw_tables(const cgtp_plan_s*) {}
void free_uvuv_tables(const cgtp_plan_s*) {}
void free_radial_maps(const cgtp_plan_s*) {}
void free_linear_tables(const cgtp_linear_s*) {}
}  // namespace cgtp

int main(int argc, char** argv) {
  for (int i = 1; i + 3 < argc; i += 4) {
    const std::string opts = argv[i + 3];  // mode/select/collapse, e.g. "uvu/all/0"
    const size_t a = opts.find('/'), b = opts.rfind('/');
    const std::string mode = opts.substr(0, a);
    const int sel = std::atoi(opts.substr(a + 1, b - a - 1).c_str());
    const bool col = opts.substr(b + 1) == "1";
    for (cgtp_dtype dt : {CGTP_F32, CGTP_F64, CGTP_BF16}) {
      for (cgtp_wkind wk : {CGTP_W_SHARED, CGTP_W_PER_ROW}) {
        try {
          cgtp_plan_s* p = cgtp::build_plan(argv[i], argv[i + 1], argv[i + 2], mode.c_str(), dt, wk,
                                            cgtp_paths(sel), col);
          std::printf("ok %d %d %lld %lld %lld %lld %zu\n", int(dt), int(wk), (long long)p->dim_x,
                      (long long)p->dim_y, (long long)p->dim_out, (long long)p->w_numel, p->paths.size());
          cgtp::destroy_plan(p);
        } catch (const cgtp::Error& e) {
          std::printf("err %d %d %d\n", int(dt), int(wk), int(e.code));
        }
      }
    }
  }
  return 0;
}
