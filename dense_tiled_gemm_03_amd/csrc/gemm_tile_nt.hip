// placeholder: replaced by the tuned kernel
#include "common.hpp"
namespace tg {
namespace {
bool accepts(Op, const GemmArgs&) { return false; }
hipError_t launch(Op, const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace
const Variant* variant_tile_nt16() {
  static const Variant v = {"tile_nt", accepts, launch};
  return &v;
}
}  // namespace tg
