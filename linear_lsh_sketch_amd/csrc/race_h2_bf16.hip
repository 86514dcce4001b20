// bf16 instantiation of the head-dimension-128 launch sequences.
#include "race_h2.hpp"

namespace race {
template race_status_t dispatch_h2<false>(const Shape&, const Derived&, const WsLayout&, const Call&);
}
